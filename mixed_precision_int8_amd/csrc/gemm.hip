// int8 GEMM of the LLM.int8() forward on gfx950 with the dequantization and the
// 16-bit outlier product fused into its epilogue.
//
//   C[t,n]  = sum_k Xq[t,k] * Wq[n,k]                 (v_mfma_i32_32x32x32_i8)
//   Y[t,n]  = fp16( C[t,n] * a[t] * b[n] / 127^2
//                   + sum_j Xo[t,j] * Wd[n,j] )       (v_mfma_f32_32x32x16_f16)
//
// "Hugging Face Quantization with bitsandbytes: 4-bit & 8-bit Models
// Explained", section 2: the non-outlier part is multiplied in int8 and
// converted back to 16-bit at the end; the outlier feature dimensions are
// multiplied in 16-bit. "bitsandbytes: GPU-Accelerated Inference and Training
// at Lower Bit Depths", "How LLM.int8() quantizes weights and activations":
// vector-wise scales (one per row of X, one per output row of W).
//
// Design (CDNA4): a workgroup of 4 or 8 wavefronts owns a BN x BT output tile
// (BN along N, BT along T); each wavefront keeps its (BN/WAVES_N) x
// (BT/WAVES_T) int32 accumulators in registers as 32x32 MFMA blocks
// (v_mfma_i32_32x32x32_i8 runs at twice the int8 rate of the 16x16x64 form on
// gfx950). Both operands are K-contiguous, the natural MFMA layout. K-stages
// of BK bytes are copied global->LDS with buffer_load_dwordx4 ... lds (no VGPR
// staging) into a ring of NSTAGE buffers, NSTAGE-1 stages in flight; rows and
// K beyond the matrix read as zero through the buffer range check. The ring is
// synchronised with partial vmcnt waits and a fence-free s_barrier, so the
// prefetch is never drained. LDS rows carry an XOR swizzle of their 16-byte
// chunks chosen so that the fragment reads (ds_read_b128) are bank-conflict
// free. Blocks are remapped so that each XCD (own L2) works on a contiguous
// range of tiles sharing weight rows.
#include "device_util.h"
#include "internal.h"

namespace llmint8 {

template <int BN_, int BT_, int BK_, int NSTAGE_, int WAVES_N_, int WAVES_T_>
struct GemmTile {
  static constexpr int BN = BN_, BT = BT_, BK = BK_, NSTAGE = NSTAGE_;
  static constexpr int WAVES_N = WAVES_N_, WAVES_T = WAVES_T_;
  static constexpr int NWAVES = WAVES_N * WAVES_T;
  static constexpr int kThreads = 64 * NWAVES;
  static constexpr int WN = BN / WAVES_N, WT = BT / WAVES_T;
  static constexpr int FN = WN / 32, FT = WT / 32;  // 32x32 MFMA blocks per wavefront
  static constexpr int KS = BK / 32;        // MFMA k-steps (32 bytes) per stage
  static constexpr int CPR = BK / 16;       // 16-byte chunks per LDS row
  static constexpr int RPB = 64 / CPR;      // rows per 1 KB direct-to-LDS issue
  static constexpr int A_BYTES = BN * BK, B_BYTES = BT * BK;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS = STAGE * NSTAGE;
  static constexpr int A_ISSUES = BN / RPB / NWAVES;
  static constexpr int B_ISSUES = BT / RPB / NWAVES;
  static constexpr int LOADS = A_ISSUES + B_ISSUES;  // vmcnt per stage per wavefront
  static_assert(BN % (RPB * NWAVES) == 0 && BT % (RPB * NWAVES) == 0, "issue split");
  static_assert(WN % 32 == 0 && WT % 32 == 0 && (BK == 64 || BK == 128), "tile shape");
  static_assert((NSTAGE - 2) * LOADS < 64, "vmcnt range");
  static_assert(LDS <= 160 * 1024, "LDS");
};

// 16-byte chunk swizzle of an LDS row: physical chunk = logical ^ swz(row).
// It depends on the row index mod 32 only (a fragment row is known mod 32 on
// the read side). With it, the 32 rows x 2 chunks that one ds_read_b128 of a
// 32x32 MFMA fragment touches are spread over all banks (measured
// conflict-free on gfx950 for both 64- and 128-byte rows).
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  r &= 31;
  return (r ^ (r >> 3)) & (CPR - 1);
}

__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// s_waitcnt vmcnt(n) (gfx9 encoding; expcnt/lgkmcnt left at their maximum)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without the memory fence of __syncthreads(): the fence would
// wait for every outstanding load (vmcnt(0)) and drain the global->LDS pipeline.
// Ordering of the LDS data is given by the explicit vmcnt waits before it; the
// "memory" clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

template <class G>
__global__ __launch_bounds__(G::kThreads, 1) void kb_gemm(LinearArgs a, int tiles_t, int group_n) {
  __shared__ __attribute__((aligned(1024))) char smem[G::LDS + (G::BN + G::BT) * 4];
  // the tile's weight and activation scales, read by the epilogue
  float* sW_l = reinterpret_cast<float*>(smem + G::LDS);
  float* aX_l = sW_l + G::BN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % G::WAVES_N, wt = wave / G::WAVES_N;

  // Tile order. Hardware deals blocks round-robin over the 8 XCDs; each XCD
  // gets a contiguous run of tile ids. Ids are then grouped: group_n weight
  // row-blocks (n) sweep all activation blocks (t) with n fastest, so the
  // tiles an XCD runs concurrently share a few weight and activation panels
  // and most K-slices are hits in that XCD's L2.
  const int nb = gridDim.x, b = blockIdx.x;
  const int nb8 = nb & ~7;
  const int id = b < nb8 ? (b & 7) * (nb8 >> 3) + (b >> 3) : b;
  const int tiles_n = (a.N + G::BN - 1) / G::BN;
  const int per_group = group_n * tiles_t;
  const int grp = id / per_group, in_grp = id % per_group;
  const int gn = min(group_n, tiles_n - grp * group_n);
  const int tile_n = grp * group_n + in_grp % gn;
  const int tile_t = in_grp / gn;

  const int K = a.K, N = a.N, T = a.T;
  const int n0 = tile_n * G::BN, t0 = tile_t * G::BT;
  const int rows_n = min(G::BN, N - n0), rows_t = min(G::BT, T - t0);
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(a.Wq + (size_t)n0 * K, (uint32_t)(rows_n * K));
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(a.Xq + (size_t)t0 * K, (uint32_t)(rows_t * K));

  // global->LDS: issue i of this wavefront fills 1 KB block (i*NWAVES + wave),
  // i.e. RPB rows x CPR chunks; lane -> physical (row, chunk), loading the
  // logical chunk that the swizzle places there.
  const int pr = lane / G::CPR, pc = lane % G::CPR;
  uint32_t offA[G::A_ISSUES], offB[G::B_ISSUES];
  int kcA[G::A_ISSUES], kcB[G::B_ISSUES];
#pragma unroll
  for (int i = 0; i < G::A_ISSUES; ++i) {
    const int row = (i * G::NWAVES + wave) * G::RPB + pr;
    kcA[i] = (pc ^ swz<G::CPR>(row)) * 16;
    offA[i] = (uint32_t)(row * K + kcA[i]);
  }
#pragma unroll
  for (int i = 0; i < G::B_ISSUES; ++i) {
    const int row = (i * G::NWAVES + wave) * G::RPB + pr;
    kcB[i] = (pc ^ swz<G::CPR>(row)) * 16;
    offB[i] = (uint32_t)(row * K + kcB[i]);
  }

  auto issue = [&](int slot, int kt) {
    const int kb = kt * G::BK;
    char* sA = smem + slot * G::STAGE;
    char* sB = sA + G::A_BYTES;
    const bool full = kb + G::BK <= K;
#pragma unroll
    for (int i = 0; i < G::A_ISSUES; ++i)
      lds_dma16(rA, sA + (i * G::NWAVES + wave) * 1024,
                (full || kb + kcA[i] < K) ? offA[i] + kb : kOobOffset);
#pragma unroll
    for (int i = 0; i < G::B_ISSUES; ++i)
      lds_dma16(rB, sB + (i * G::NWAVES + wave) * 1024,
                (full || kb + kcB[i] < K) ? offB[i] + kb : kOobOffset);
  };

  // MFMA operand addressing: lane (i = lane&31, g = lane>>5) holds 16 bytes of
  // fragment row i at logical chunk 2*ks+g; every fragment row is i mod 32.
  const int fi = lane & 31, fg = lane >> 5;
  const int fswz = swz<G::CPR>(fi);
  int aoff[G::KS], boff[G::KS];
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks) {
    const int phys = (ks * 2 + fg) ^ fswz;
    aoff[ks] = (wn * G::WN + fi) * G::BK + phys * 16;
    boff[ks] = G::A_BYTES + (wt * G::WT + fi) * G::BK + phys * 16;
  }
  struct Frags { v4i a[G::FN], b[G::FT]; };
  auto read_frags = [&](Frags& f, int slot, int ks) {
    const char* st = smem + slot * G::STAGE;
#pragma unroll
    for (int j = 0; j < G::FT; ++j) f.b[j] = *reinterpret_cast<const v4i*>(st + boff[ks] + j * 32 * G::BK);
#pragma unroll
    for (int i = 0; i < G::FN; ++i) f.a[i] = *reinterpret_cast<const v4i*>(st + aoff[ks] + i * 32 * G::BK);
  };

  v16i acc[G::FN][G::FT];
#pragma unroll
  for (int i = 0; i < G::FN; ++i)
#pragma unroll
    for (int j = 0; j < G::FT; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;
  auto mfma = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < G::FN; ++i)
#pragma unroll
      for (int j = 0; j < G::FT; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
  };
  // keep the next k-step's fragment reads ahead of this k-step's MFMAs
  auto order_reads_before_mfma = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, G::FN + G::FT, 0);  // DS reads
    __builtin_amdgcn_sched_group_barrier(0x008, G::FN * G::FT, 0);  // MFMAs
  };

  constexpr int P = G::NSTAGE - 1;  // stages in flight ahead of the one computed
  static_assert(G::KS % 2 == 0, "fragment double buffer alternates per k-step");
  // Software pipeline. The fragments of k-step s+1 are read from LDS while
  // the MFMAs of k-step s run; at the end of a stage each wavefront waits for
  // the next stage's copy and for its own LDS reads, then the workgroup
  // barrier. The loop is rotated so that an iteration starts right after that
  // barrier (no LDS read outstanding across the back-edge, so the compiler's
  // wait counts stay exact) and it is branch-free: stages past the end are
  // still issued, as out-of-range loads that write zeros into a slot nobody
  // reads again.
  const int KT = (K + G::BK - 1) / G::BK;
  Frags f0, f1;
  // one stage: reads of k-step 0 of stage `slot`, the last k-step's MFMAs of
  // the previous stage (if any), then the rest; ends after the barrier.
  auto stage = [&](int slot, int kt, bool has_prev) {
    const int next_slot = slot == P ? 0 : slot + 1;
    read_frags(f0, slot, 0);
    if (has_prev) {
      mfma(f1);
      order_reads_before_mfma();
    }
    // refill the slot of stage kt-1: every wavefront has passed the barrier
    // that followed its last reads of that stage
    issue(slot == 0 ? P : slot - 1, kt + P);
#pragma unroll
    for (int ks = 1; ks < G::KS; ++ks) {
      Frags& cur = (ks & 1) ? f0 : f1;   // holds k-step ks-1
      Frags& nxt = (ks & 1) ? f1 : f0;   // receives k-step ks
      read_frags(nxt, slot, ks);
      mfma(cur);
      order_reads_before_mfma();
    }
    // stage kt+1 must have landed (later stages may still be in flight) and
    // this wavefront's reads of stage kt must be done before the barrier.
    // The scheduling barrier keeps this stage's MFMAs ahead of the waits, so
    // they run while the copy lands.
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<(P - 1) * G::LOADS>();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    barrier_no_fence();
    (void)next_slot;
  };
  {
    // scales -> LDS by direct copy (rows past the matrix read as zero). They
    // are issued before the first K stage, so the stage waits cover them.
    constexpr int CS = (G::BN + 63) / 64, CX = (G::BT + 63) / 64;
    const __amdgpu_buffer_rsrc_t rS = make_rsrc(a.sW + n0, (uint32_t)(rows_n * 4));
    const __amdgpu_buffer_rsrc_t rX = make_rsrc(a.aX + t0, (uint32_t)(rows_t * 4));
    for (int c = wave; c < CS + CX; c += G::NWAVES) {
      const bool is_w = c < CS;  // wave-uniform
      const int cc = is_w ? c : c - CS;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          is_w ? rS : rX, (__attribute__((address_space(3))) void*)((is_w ? sW_l : aX_l) + cc * 64),
          4, (uint32_t)((cc * 64 + lane) * 4), 0, 0, 0);
    }
  }
#pragma unroll
  for (int s = 0; s < P; ++s) issue(s, s);
  wait_vmcnt<(P - 1) * G::LOADS>();
  barrier_no_fence();
  stage(0, 0, false);
  int slot = 1 % G::NSTAGE;
  for (int kt = 1; kt < KT; ++kt) {
    stage(slot, kt, true);
    slot = slot == P ? 0 : slot + 1;
  }
  mfma(f1);  // last k-step of the last stage

  // ---- epilogue, one 32-row block of n at a time. Output layout of a 32x32
  // block: lane holds, for column (t) lane&31, rows (n) 8*q + 4*(lane>>5) + r
  // in register 4*q + r (q, r = 0..3).
  const int nl = n0 + wn * G::WN + 4 * fg;  // + i*32 + 8*q + r
  const int tl = t0 + wt * G::WT + fi;      // + j*32
  float as[G::FT];
#pragma unroll
  for (int j = 0; j < G::FT; ++j) as[j] = aX_l[wt * G::WT + fi + j * 32];
  const bool vec_ok = (N & 3) == 0;
  const int count = *a.count;
  const int nch = (count + kOutChunk - 1) / kOutChunk;
  // Operands of the first chunk of 32 outlier columns (the common case is a
  // single chunk), all requested before the first is used so that the
  // epilogue pays one memory latency rather than one per block.
  v8h wf0[G::FN][2], xf0[G::FT][2];
  if (nch > 0) {
#pragma unroll
    for (int i = 0; i < G::FN; ++i) {
      const int nrow = min(n0 + wn * G::WN + i * 32 + fi, N - 1);
#pragma unroll
      for (int h = 0; h < 2; ++h)
        wf0[i][h] = *reinterpret_cast<const v8h*>(a.Wd + (size_t)nrow * kOutChunk + h * 16 + fg * 8);
    }
#pragma unroll
    for (int j = 0; j < G::FT; ++j) {
      const int t = min(tl + j * 32, T - 1);
#pragma unroll
      for (int h = 0; h < 2; ++h)
        xf0[j][h] = *reinterpret_cast<const v8h*>(a.Xo + (size_t)t * kOutChunk + h * 16 + fg * 8);
    }
  }
#pragma unroll
  for (int i = 0; i < G::FN; ++i) {
    float bs[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const v4f w4 = *reinterpret_cast<const v4f*>(sW_l + wn * G::WN + 4 * fg + i * 32 + 8 * q);
#pragma unroll
      for (int r = 0; r < 4; ++r) bs[4 * q + r] = w4[r] * (1.0f / 16129.0f);
    }
    if (a.dbg_C) {
#pragma unroll
      for (int j = 0; j < G::FT; ++j) {
        const int t = tl + j * 32;
        if (t >= T) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int n = nl + i * 32 + 8 * (v >> 2) + (v & 3);
          if (n < N) a.dbg_C[(size_t)t * N + n] = acc[i][j][v];
        }
      }
    }
    v16f y[G::FT];
#pragma unroll
    for (int j = 0; j < G::FT; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) y[j][v] = (float)acc[i][j][v] * (as[j] * bs[v]);
    // outlier columns: fp16 operands, fp32 accumulation on top of the int8 part;
    // a chunk of 32 outlier columns is two 32x32x16 steps.
    if (nch > 0) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < G::FT; ++j)
          y[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf0[i][h], xf0[j][h], y[j], 0, 0, 0);
    }
    const int nrow = min(n0 + wn * G::WN + i * 32 + fi, N - 1);
    for (int c = 1; c < nch; ++c) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const v8h wf = *reinterpret_cast<const v8h*>(
            a.Wd + ((size_t)c * N + nrow) * kOutChunk + h * 16 + fg * 8);
#pragma unroll
        for (int j = 0; j < G::FT; ++j) {
          const int t = min(tl + j * 32, T - 1);
          const v8h xf = *reinterpret_cast<const v8h*>(
              a.Xo + ((size_t)c * T + t) * kOutChunk + h * 16 + fg * 8);
          y[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf, xf, y[j], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < G::FT; ++j) {
      const int t = tl + j * 32;
      if (t >= T) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = nl + i * 32 + 8 * q;
        uint16_t* dst = a.Y + (size_t)t * N + n;
        if (vec_ok && n + 3 < N) {
          uint2 p;
          p.x = (uint32_t)float_to_half_bits(y[j][4 * q]) |
                ((uint32_t)float_to_half_bits(y[j][4 * q + 1]) << 16);
          p.y = (uint32_t)float_to_half_bits(y[j][4 * q + 2]) |
                ((uint32_t)float_to_half_bits(y[j][4 * q + 3]) << 16);
          *reinterpret_cast<uint2*>(dst) = p;
        } else {
          for (int r = 0; r < 4; ++r)
            if (n + r < N) dst[r] = float_to_half_bits(y[j][4 * q + r]);
        }
      }
    }
  }
}

template <class G>
hipError_t launch_gemm_tile(const LinearArgs& a, hipStream_t stream, int group_n) {
  const int tn = (a.N + G::BN - 1) / G::BN, tt = (a.T + G::BT - 1) / G::BT;
  if (group_n < 1) group_n = 1;
  hipLaunchKernelGGL(kb_gemm<G>, dim3(tn * tt), dim3(G::kThreads), 0, stream, a, tt, group_n);
  return hipGetLastError();
}

// Tile shapes (BN x BT, BK, LDS stages, wavefronts along N x T).
using Tile256x256 = GemmTile<256, 256, 128, 2, 2, 4>;  // 8 wavefronts of 128x64
using Tile192x256 = GemmTile<192, 256, 128, 2, 2, 4>;  // 8 wavefronts of 96x64
using Tile256x128 = GemmTile<256, 128, 128, 2, 2, 4>;  // 8 wavefronts of 128x32
using Tile128x128 = GemmTile<128, 128, 128, 4, 2, 2>;  // 4 wavefronts of 64x64

constexpr int kGroupN = 8;  // weight row-blocks per rasterization group

// Tile choice: minimise (rounds of CUs) x (time per tile), where a tile's
// time is its MFMA work divided by a per-shape efficiency (measured on gfx950:
// smaller tiles move more operand bytes per MFMA and run less efficiently).
hipError_t launch_gemm(const LinearArgs& a, int num_cus, hipStream_t stream) {
  struct Cand { int bn, bt; double eff; };
  const Cand cands[] = {{256, 256, 1.0}, {192, 256, 0.93}, {256, 128, 0.8}, {128, 128, 0.55}};
  int best = 0;
  double best_cost = 1e300;
  for (int i = 0; i < 4; ++i) {
    const double tiles = (double)ceil_div(a.N, cands[i].bn) * (double)ceil_div(a.T, cands[i].bt);
    const double rounds = std::ceil(tiles / num_cus);
    const double cost = rounds * cands[i].bn * cands[i].bt / cands[i].eff;
    if (cost < best_cost * 0.999) { best_cost = cost; best = i; }
  }
  switch (best) {
    case 0: return launch_gemm_tile<Tile256x256>(a, stream, kGroupN);
    case 1: return launch_gemm_tile<Tile192x256>(a, stream, kGroupN);
    case 2: return launch_gemm_tile<Tile256x128>(a, stream, kGroupN);
    default: return launch_gemm_tile<Tile128x128>(a, stream, kGroupN);
  }
}

}  // namespace llmint8
