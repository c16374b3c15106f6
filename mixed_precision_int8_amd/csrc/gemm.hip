// int8 GEMM of the LLM.int8() forward on gfx950 with the dequantization and the
// 16-bit outlier product fused into its epilogue.
//
//   C[t,n]  = sum_k Xq[t,k] * Wq[n,k]                 (v_mfma_i32_16x16x64_i8)
//   Y[t,n]  = fp16( C[t,n] * a[t] * b[n] / 127^2
//                   + sum_j Xo[t,j] * Wd[n,j] )       (v_mfma_f32_16x16x32_f16)
//
// "Hugging Face Quantization with bitsandbytes: 4-bit & 8-bit Models
// Explained", section 2: the non-outlier part is multiplied in int8 and
// converted back to 16-bit at the end; the outlier feature dimensions are
// multiplied in 16-bit. "bitsandbytes: GPU-Accelerated Inference and Training
// at Lower Bit Depths", "How LLM.int8() quantizes weights and activations":
// vector-wise scales (one per row of X, one per output row of W).
//
// Design (CDNA4): a 256-thread workgroup (2x2 wavefronts) owns a BN x BT output
// tile (BN along N, BT along T). Both operands are K-contiguous, the natural
// MFMA layout. Each K-stage of 128 bytes is copied global->LDS with
// buffer_load_dwordx4 ... lds (no VGPR staging), double buffered; rows and K
// beyond the matrix read as zero through the buffer range check. LDS rows are
// 128 bytes with a per-row XOR swizzle of the 16-byte chunks, so the MFMA
// operand reads (ds_read_b128, 16 rows per lane group) hit distinct banks.
// Each wavefront keeps a (BN/2) x (BT/2) int32 accumulator tile in registers.
// Blocks are remapped so that each XCD (own L2) works on a contiguous range of
// tiles sharing weight rows.
#include "device_util.h"
#include "internal.h"

namespace llmint8 {

template <int BN_, int BT_>
struct GemmTile {
  static constexpr int BN = BN_, BT = BT_;
  static constexpr int kThreads = 256;
  static constexpr int BK = 128;  // bytes of K per stage
  static constexpr int WN = BN / 2, WT = BT / 2;
  static constexpr int FN = WN / 16, FT = WT / 16;
  static constexpr int A_BYTES = BN * BK, B_BYTES = BT * BK;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int NSTAGE = 2;
  static constexpr int LDS = STAGE * NSTAGE;
  static constexpr int A_ISSUES = BN / 32;  // 1 KB (8-row) blocks per wavefront
  static constexpr int B_ISSUES = BT / 32;
};

// 16-byte chunk swizzle for 128-byte LDS rows: rows r and r' in the same group
// of 8 (and, for 64-bank reads, of 16 with different parity) never share a chunk.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

template <class G>
__global__ __launch_bounds__(256, 1) void kb_gemm(LinearArgs a, int tiles_t) {
  __shared__ __attribute__((aligned(1024))) char smem[G::LDS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wt = wave >> 1;

  // XCD-aware order: hardware deals blocks round-robin over 8 XCDs.
  const int nb = gridDim.x, b = blockIdx.x;
  const int nb8 = nb & ~7;
  const int id = b < nb8 ? (b & 7) * (nb8 >> 3) + (b >> 3) : b;
  const int tile_t = id % tiles_t, tile_n = id / tiles_t;

  const int K = a.K, N = a.N, T = a.T;
  const int n0 = tile_n * G::BN, t0 = tile_t * G::BT;
  const int rows_n = min(G::BN, N - n0), rows_t = min(G::BT, T - t0);
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(a.Wq + (size_t)n0 * K, (uint32_t)(rows_n * K));
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(a.Xq + (size_t)t0 * K, (uint32_t)(rows_t * K));

  // global->LDS mapping: a wavefront fills 1 KB = 8 rows x 8 chunks per issue;
  // lane -> physical (row lr, chunk pc); it loads logical chunk pc ^ swz(row).
  const int lr = lane >> 3, pc = lane & 7;
  const int lchunk = pc ^ (lr ^ (wave & 1));  // swz of row (blk*8+lr), blk parity = wave parity
  const uint32_t coff = (uint32_t)lchunk * 16u;
  uint32_t rowA[G::A_ISSUES], rowB[G::B_ISSUES];
#pragma unroll
  for (int i = 0; i < G::A_ISSUES; ++i) rowA[i] = (uint32_t)((i * 32 + wave * 8 + lr) * K);
#pragma unroll
  for (int i = 0; i < G::B_ISSUES; ++i) rowB[i] = (uint32_t)((i * 32 + wave * 8 + lr) * K);

  auto issue = [&](int stage, int kt) {
    const int kb = kt * G::BK;
    const bool ok = (int)(kb + coff) < K;
    char* sA = smem + stage * G::STAGE;
    char* sB = sA + G::A_BYTES;
#pragma unroll
    for (int i = 0; i < G::A_ISSUES; ++i)
      lds_dma16(rA, sA + (i * 4 + wave) * 1024, ok ? rowA[i] + kb + coff : kOobOffset);
#pragma unroll
    for (int i = 0; i < G::B_ISSUES; ++i)
      lds_dma16(rB, sB + (i * 4 + wave) * 1024, ok ? rowB[i] + kb + coff : kOobOffset);
  };

  // MFMA operand addressing: lane (i = lane&15, g = lane>>4) holds 16 bytes of
  // row i at logical chunk ks*4+g. Row r%16 == i for every fragment row.
  const int fi = lane & 15, fg = lane >> 4;
  const int fswz = swz(fi);
  int aoff[2], boff[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int phys = (ks * 4 + fg) ^ fswz;
    aoff[ks] = (wn * G::WN + fi) * G::BK + phys * 16;
    boff[ks] = G::A_BYTES + (wt * G::WT + fi) * G::BK + phys * 16;
  }

  v4i acc[G::FN][G::FT];
#pragma unroll
  for (int i = 0; i < G::FN; ++i)
#pragma unroll
    for (int j = 0; j < G::FT; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  const int KT = (K + G::BK - 1) / G::BK;
  issue(0, 0);
  for (int kt = 0; kt < KT; ++kt) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (kt + 1 < KT) issue((kt + 1) & 1, kt + 1);
    const char* st = smem + (kt & 1) * G::STAGE;
    // all operand fragments of the stage first (2 k-steps), then the MFMAs;
    // the scheduling barriers keep the compiler from serialising the reads.
    v4i af[2][G::FN], bf[2][G::FT];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int j = 0; j < G::FT; ++j)
        bf[ks][j] = *reinterpret_cast<const v4i*>(st + boff[ks] + j * 16 * G::BK);
#pragma unroll
      for (int i = 0; i < G::FN; ++i)
        af[ks][i] = *reinterpret_cast<const v4i*>(st + aoff[ks] + i * 16 * G::BK);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < G::FN; ++i)
#pragma unroll
        for (int j = 0; j < G::FT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[ks][i], bf[ks][j], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * (G::FN + G::FT), 0);  // DS reads
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * G::FN * G::FT, 0);     // MFMAs
  }

  // ---- epilogue, one 16-row block of n at a time (keeps register use low).
  // Output layout of a 16x16 block: lane holds rows (n) 4*(lane>>4)+v, v=0..3,
  // of column (t) lane&15.
  const int nl = n0 + wn * G::WN + 4 * fg;  // + i*16 + v
  const int tl = t0 + wt * G::WT + fi;      // + j*16
  float as[G::FT];
#pragma unroll
  for (int j = 0; j < G::FT; ++j) {
    const int t = tl + j * 16;
    as[j] = t < T ? a.aX[t] : 0.0f;
  }
  const bool vec_ok = (N & 3) == 0;
  const int count = *a.count;
  const int nch = (count + kOutChunk - 1) / kOutChunk;
#pragma unroll
  for (int i = 0; i < G::FN; ++i) {
    const int n = nl + i * 16;  // first of this lane's 4 rows
    float bs[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) bs[v] = n + v < N ? a.sW[n + v] * (1.0f / 16129.0f) : 0.0f;
    if (a.dbg_C) {
#pragma unroll
      for (int j = 0; j < G::FT; ++j) {
        const int t = tl + j * 16;
        if (t < T) {
          int32_t* dst = a.dbg_C + (size_t)t * N + n;
          for (int v = 0; v < 4; ++v)
            if (n + v < N) dst[v] = acc[i][j][v];
        }
      }
    }
    v4f y[G::FT];
#pragma unroll
    for (int j = 0; j < G::FT; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) y[j][v] = (float)acc[i][j][v] * (as[j] * bs[v]);
    // outlier columns: fp16 operands, fp32 accumulation on top of the int8 part
    const int nrow = min(n0 + wn * G::WN + i * 16 + fi, N - 1);
    for (int c = 0; c < nch; ++c) {
      const v8h wf = *reinterpret_cast<const v8h*>(a.Wd + ((size_t)c * N + nrow) * kOutChunk + fg * 8);
#pragma unroll
      for (int j = 0; j < G::FT; ++j) {
        const int t = min(tl + j * 16, T - 1);
        const v8h xf = *reinterpret_cast<const v8h*>(a.Xo + ((size_t)c * T + t) * kOutChunk + fg * 8);
        y[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf, xf, y[j], 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < G::FT; ++j) {
      const int t = tl + j * 16;
      if (t >= T) continue;
      uint16_t* dst = a.Y + (size_t)t * N + n;
      if (vec_ok && n + 3 < N) {
        uint2 p;
        p.x = (uint32_t)float_to_half_bits(y[j][0]) | ((uint32_t)float_to_half_bits(y[j][1]) << 16);
        p.y = (uint32_t)float_to_half_bits(y[j][2]) | ((uint32_t)float_to_half_bits(y[j][3]) << 16);
        *reinterpret_cast<uint2*>(dst) = p;
      } else {
        for (int v = 0; v < 4; ++v)
          if (n + v < N) dst[v] = float_to_half_bits(y[j][v]);
      }
    }
  }
}

template <class G>
static hipError_t launch_tile(const LinearArgs& a, hipStream_t stream) {
  const int tn = (a.N + G::BN - 1) / G::BN, tt = (a.T + G::BT - 1) / G::BT;
  hipLaunchKernelGGL(kb_gemm<G>, dim3(tn * tt), dim3(G::kThreads), 0, stream, a, tt);
  return hipGetLastError();
}

// Tile choice: minimise (rounds of 256 CUs) x (time per tile), with smaller
// tiles charged for their lower operand reuse.
hipError_t launch_gemm(const LinearArgs& a, int num_cus, hipStream_t stream) {
  struct Cand { int bn, bt; double eff; };
  const Cand cands[] = {{256, 256, 1.0}, {256, 128, 0.9}, {128, 128, 0.7}};
  int best = 0;
  double best_cost = 1e300;
  for (int i = 0; i < 3; ++i) {
    const double tiles = (double)ceil_div(a.N, cands[i].bn) * (double)ceil_div(a.T, cands[i].bt);
    const double rounds = std::ceil(tiles / num_cus);
    const double cost = rounds * cands[i].bn * cands[i].bt / cands[i].eff;
    if (cost < best_cost * 0.999) { best_cost = cost; best = i; }
  }
  switch (best) {
    case 0: return launch_tile<GemmTile<256, 256>>(a, stream);
    case 1: return launch_tile<GemmTile<256, 128>>(a, stream);
    default: return launch_tile<GemmTile<128, 128>>(a, stream);
  }
}

}  // namespace llmint8
