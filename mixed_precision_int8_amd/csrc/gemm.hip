// int8 GEMM of the LLM.int8() forward on gfx950 with the dequantization and the
// 16-bit outlier product fused into its epilogue.
//
//   C[t,n]  = sum_k Xq[t,k] * Wq[n,k]                 (v_mfma_i32_32x32x32_i8)
//   Y[t,n]  = r16( C[t,n] * a[t] * b[n] / 127^2
//                  + sum_j Xo[t,j] * Wd[n,j] + bias[n] )
//             (v_mfma_f32_32x32x16_f16 / _bf16; r16 rounds to the activation
//              type, fp16 or bf16, and the bias is optional)
//
// "Hugging Face Quantization with bitsandbytes: 4-bit & 8-bit Models
// Explained", section 2: the non-outlier part is multiplied in int8 and
// converted back to 16-bit at the end; the outlier feature dimensions are
// multiplied in 16-bit. "bitsandbytes: GPU-Accelerated Inference and Training
// at Lower Bit Depths", "How LLM.int8() quantizes weights and activations":
// vector-wise scales (one per row of X, one per output row of W).
//
// Design (CDNA4): a workgroup of 4 or 8 wavefronts owns a BN x BT output tile
// (BN along N, BT along T); each wavefront keeps its share of the int32
// accumulators in registers as 32x32 MFMA blocks (v_mfma_i32_32x32x32_i8 runs
// at twice the int8 rate of the 16x16x64 form on gfx950). Both operands are
// K-contiguous, the natural MFMA layout; the K loops (direct-to-LDS copy ring,
// swizzled fragments, XCD-aware tile order) are those of gemm_common.h, with
// Wq rows as A and Xq rows as B. kb_gemm takes the evenly split tiles;
// kb_gemm_split the 352 x 256 tile, whose 11 row blocks split 6 + 5 over the
// two wavefront columns, so that 256 tiles of it cover a 2048 x 11008 output
// in one round of the 256 CUs.
#include "gemm_common.h"

namespace llmint8 {

// 16-bit outlier operands of outliers j0 .. j0+7 (zero past |O|) for a chunk
// the workspace does not hold: formed from Wq and X exactly as the prepare
// kernel forms Wd and Xo, Wd[n,j] = r16(fl32(fl32(Wq[n,idx_j] * b_n) / 127)).
template <bool BF16>
__device__ __forceinline__ uint4 outlier_w8(const LinearArgs& a, int n, int j0, int count) {
  const float b = a.sW[n];
  const int8_t* wr = a.Wq + (size_t)n * a.K;
  uint32_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    v[e] = j0 + e < count ? Act16<BF16>::from_f32(((float)wr[a.idx[j0 + e]] * b) / 127.0f) : 0u;
  return make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16));
}
__device__ __forceinline__ uint4 outlier_x8(const LinearArgs& a, int t, int j0, int count) {
  const uint16_t* xr = a.X + (size_t)t * a.K;
  uint32_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = j0 + e < count ? (uint32_t)xr[a.idx[j0 + e]] : 0u;
  return make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16));
}

// The LDS layout of staged outlier operands: a chunk of 32 outlier columns is
// BN rows of Wd then BT rows of Xo, 64 bytes each; row r keeps its 16-byte
// piece c at position c ^ ((r >> 2) & 3), so that the epilogue's reads (32 rows
// x 2 pieces per instruction) are free of bank conflicts.
__device__ __forceinline__ uint4 staged_outlier_piece(const char* area, int r, int piece) {
  return *reinterpret_cast<const uint4*>(area + r * 64 + ((piece ^ ((r >> 2) & 3)) * 16));
}

// Direct copies of chunk c's operands of the tile (rows past the matrix read
// as zero) into `area`; every wavefront of the block takes pieces of 1 KB
// (16 rows) in turn.
template <int BN, int BT, int NWAVES>
__device__ __forceinline__ void stage_outlier_chunk(const LinearArgs& a, int c, int n0, int t0, int rows_n,
                                                    int rows_t, char* area, int wave, int lane) {
  constexpr int CW = BN * 64 / 1024, CXO = BT * 64 / 1024;
  static_assert(BN * 64 % 1024 == 0 && BT * 64 % 1024 == 0, "1 KB pieces");
  const __amdgpu_buffer_rsrc_t rW =
      make_rsrc(a.Wd + ((size_t)c * a.N + n0) * kOutChunk, (uint32_t)(rows_n * 64));
  const __amdgpu_buffer_rsrc_t rO =
      make_rsrc(a.Xo + ((size_t)c * a.T + t0) * kOutChunk, (uint32_t)(rows_t * 64));
  for (int p = wave; p < CW + CXO; p += NWAVES) {
    const bool is_w = p < CW;  // wave-uniform
    const int r = p * 16 + (lane >> 2);  // row of the staged area this lane fills
    const uint32_t src = (uint32_t)((is_w ? p : p - CW) * 1024 + (lane >> 2) * 64 +
                                    (((lane & 3) ^ ((r >> 2) & 3)) * 16));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(is_w ? rW : rO,
                                             (__attribute__((address_space(3))) void*)(area + p * 1024),
                                             16, src, 0, 0, 0);
  }
}

// Where the epilogue may stage outlier chunks 1, 2, ... of a tile: `buf`, the
// block's LDS ring (free once every wavefront is past the K loop; all copies
// landed), of `bytes`; wavefront `wave` of NWAVES; tile origin and extent.
struct ChunkStaging {
  char* buf;
  int bytes, wave, n0, t0, rows_n, rows_t;
};

// Epilogue of one wavefront: its FNW x FT accumulator blocks, at rows wrow..
// (weights) and wcol.. (activations) of a BN x BT tile at (n0, t0) of the
// output. sW_w / aX_w / bias_w point at the wavefront's first entries of the
// tile's scales and bias in LDS (bias_w null without bias). `wf(i, h)` /
// `xf(j, h)` give the 16-bit operands of the first chunk of 32 outlier columns
// (k-step h of block i / j). Output layout of a 32x32 block: lane holds, for
// column (t) lane&31, rows (n) 8*q + 4*(lane>>5) + r in register 4*q + r.
//
// Three phases. (1) Every block is dequantized, C * a * b / 127^2, and takes
// the first chunk's 16-bit product. (2) Chunks 1, 2, ... that the workspace
// holds go through LDS: all wavefronts of the block copy as many chunks as
// `cs.buf` holds, wait, multiply every block with them and wait again, so
// each chunk costs one memory latency per tile. Chunks past those the
// workspace holds are formed from X and Wq per block. (3) Bias, rounding and
// the store of each block. Every wavefront of a block calls this with the
// same |O| (the barriers of phase 2 are the block's).
//
// Y is written one of two ways. Directly, each lane stores its 4-value pieces
// (16 contiguous bytes of an output row per instruction). Or, when `stage`
// (a wavefront-private LDS area of kStageBytes) is given, the tile lies wholly
// inside Y and rows are 16-byte aligned, through LDS: two 32-row blocks are
// gathered as 64 output rows of 128 bytes and stored as whole 128-byte lines.
template <bool BF16, int FNW, int FT, int BN, int BT, int NWAVES, class WF, class XF>
__device__ __forceinline__ void gemm_epilogue(const LinearArgs& a, const v16i (&acc)[FNW][FT], int wrow,
                                              int wcol, const float* sW_w, const float* aX_w,
                                              const uint16_t* bias_w, int count, int lane, WF&& wf,
                                              XF&& xf, const ChunkStaging& cs, char* stage = nullptr) {
  using A16 = Act16<BF16>;
  const int N = a.N, T = a.T;
  const int nw0 = cs.n0 + wrow, tw0 = cs.t0 + wcol;
  const int nch = (count + kOutChunk - 1) / kOutChunk;
  const int fi = lane & 31, fg = lane >> 5;
  const int nl = nw0 + 4 * fg;  // + i*32 + 8*q + r
  const int tl = tw0 + fi;      // + j*32
  float as[FT];
#pragma unroll
  for (int j = 0; j < FT; ++j) as[j] = aX_w[fi + j * 32];
  const bool vec_ok = (N & 3) == 0;

  // ---- (1) dequantization and the first outlier chunk, every block
  v16f y[FNW][FT];
#pragma unroll
  for (int i = 0; i < FNW; ++i) {
    float bs[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const v4f w4 = *reinterpret_cast<const v4f*>(sW_w + 4 * fg + i * 32 + 8 * q);
#pragma unroll
      for (int r = 0; r < 4; ++r) bs[4 * q + r] = w4[r] * (1.0f / 16129.0f);
    }
    if (a.dbg_C) {
#pragma unroll
      for (int j = 0; j < FT; ++j) {
        const int t = tl + j * 32;
        if (t >= T) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int n = nl + i * 32 + 8 * (v >> 2) + (v & 3);
          if (n < N) a.dbg_C[(size_t)t * N + n] = acc[i][j][v];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < FT; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) y[i][j][v] = (float)acc[i][j][v] * (as[j] * bs[v]);
    // outlier columns: 16-bit operands (the activation type), fp32 accumulation
    // on top of the int8 part; a chunk of 32 outlier columns is two 32x32x16 steps.
    if (nch > 0) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 w = wf(i, h);
#pragma unroll
        for (int j = 0; j < FT; ++j) y[i][j] = A16::mma32(w, xf(j, h), y[i][j]);
      }
    }
  }

  // ---- (2) chunks 1 .. held-1 through LDS, batches of as many as cs.buf holds
  const int held = min(nch, a.wchunks);
  if (held > 1) {  // uniform over the block
    constexpr int kChunkBytes = (BN + BT) * 64;
    const int per = cs.bytes / kChunkBytes;
    for (int c0 = 1; c0 < held; c0 += per) {
      const int cn = min(per, held - c0);
      wait_vmcnt<0>();
      __syncthreads();  // the ring (the K loop's, or the previous batch's) is free
      for (int cc = 0; cc < cn; ++cc)
        stage_outlier_chunk<BN, BT, NWAVES>(a, c0 + cc, cs.n0, cs.t0, cs.rows_n, cs.rows_t,
                                            cs.buf + cc * kChunkBytes, cs.wave, lane);
      wait_vmcnt<0>();
      __syncthreads();
      for (int cc = 0; cc < cn; ++cc) {
        const char* area = cs.buf + cc * kChunkBytes;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint4 x[FT];
#pragma unroll
          for (int j = 0; j < FT; ++j) x[j] = staged_outlier_piece(area, BN + wcol + j * 32 + fi, 2 * h + fg);
#pragma unroll
          for (int i = 0; i < FNW; ++i) {
            const uint4 w = staged_outlier_piece(area, wrow + i * 32 + fi, 2 * h + fg);
#pragma unroll
            for (int j = 0; j < FT; ++j) y[i][j] = A16::mma32(w, x[j], y[i][j]);
          }
        }
      }
    }
    __syncthreads();  // every wavefront's reads are done before the ring is reused
  }

  // ---- (3) chunks past the workspace (formed here), bias, rounding, stores
#pragma unroll
  for (int i = 0; i < FNW; ++i) {
    const int nrow = min(nw0 + i * 32 + fi, N - 1);
    for (int c = max(1, held); c < nch; ++c) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j0 = c * kOutChunk + h * 16 + fg * 8;
        const uint4 w = outlier_w8<BF16>(a, nrow, j0, count);
#pragma unroll
        for (int j = 0; j < FT; ++j)
          y[i][j] = A16::mma32(w, outlier_x8(a, min(tl + j * 32, T - 1), j0, count), y[i][j]);
      }
    }
    if (bias_w) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float bv = A16::to_f32(bias_w[4 * fg + i * 32 + 8 * (v >> 2) + (v & 3)]);
#pragma unroll
        for (int j = 0; j < FT; ++j) y[i][j][v] += bv;
      }
    }
    if constexpr (FT == 2) if (stage) {  // uniform; 64 staged rows
      // block i -> column half (i & 1) of the staged rows t = 32 j + fi
#pragma unroll
      for (int j = 0; j < FT; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint2 p;
          p.x = (uint32_t)A16::from_f32(y[i][j][4 * q]) | ((uint32_t)A16::from_f32(y[i][j][4 * q + 1]) << 16);
          p.y = (uint32_t)A16::from_f32(y[i][j][4 * q + 2]) | ((uint32_t)A16::from_f32(y[i][j][4 * q + 3]) << 16);
          stage_put(stage, i, j, q, fi, fg, p);
        }
      if ((i & 1) || i == FNW - 1)
        stage_flush(stage, (i & 1) + 1, lane, a.Y + (size_t)tw0 * N + nw0 + (i - (i & 1)) * 32, N);
      continue;
    }
#pragma unroll
    for (int j = 0; j < FT; ++j) {
      const int t = tl + j * 32;
      if (t >= T) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = nl + i * 32 + 8 * q;
        uint16_t* dst = a.Y + (size_t)t * N + n;
        if (vec_ok && n + 3 < N) {
          uint2 p;
          p.x = (uint32_t)A16::from_f32(y[i][j][4 * q]) | ((uint32_t)A16::from_f32(y[i][j][4 * q + 1]) << 16);
          p.y = (uint32_t)A16::from_f32(y[i][j][4 * q + 2]) | ((uint32_t)A16::from_f32(y[i][j][4 * q + 3]) << 16);
          *reinterpret_cast<uint2*>(dst) = p;
        } else {
          for (int r = 0; r < 4; ++r)
            if (n + r < N) dst[r] = A16::from_f32(y[i][j][4 * q + r]);
        }
      }
    }
  }
}

// The tile's weight and activation scales -> LDS by direct copy, 64 entries per
// piece (entries past the matrix read as zero; the arrays hold whole pieces).
// Issued before the first K stage, so the stage waits cover them.
template <int BN, int BT, int NWAVES>
__device__ __forceinline__ void scales_to_lds(const LinearArgs& a, int n0, int t0, int rows_n, int rows_t,
                                              float* sW_l, float* aX_l, int wave, int lane) {
  constexpr int CS = (BN + 63) / 64, CX = (BT + 63) / 64;
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(a.sW + n0, (uint32_t)(rows_n * 4));
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(a.aX + t0, (uint32_t)(rows_t * 4));
  for (int c = wave; c < CS + CX; c += NWAVES) {
    const bool is_w = c < CS;  // wave-uniform
    const int cc = is_w ? c : c - CS;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        is_w ? rS : rX, (__attribute__((address_space(3))) void*)((is_w ? sW_l : aX_l) + cc * 64),
        4, (uint32_t)((cc * 64 + lane) * 4), 0, 0, 0);
  }
}

template <class G, bool BF16>
__global__ __launch_bounds__(G::kThreads, 1) void kb_gemm(LinearArgs a, int tiles_t, int group_n) {
  static_assert(G::BN % 64 == 0 && G::BT % 64 == 0, "whole scale pieces");
  __shared__ __attribute__((aligned(1024))) char smem[G::LDS + (G::BN + G::BT) * 4 + G::BN * 2];
  // the tile's weight and activation scales and bias, read by the epilogue
  float* sW_l = reinterpret_cast<float*>(smem + G::LDS);
  float* aX_l = sW_l + G::BN;
  uint16_t* bias_l = reinterpret_cast<uint16_t*>(aX_l + G::BT);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % G::WAVES_N, wt = wave / G::WAVES_N;

  const TileCoords tc = tile_coords<G>(a.N, tiles_t, group_n);
  const int K = a.K, N = a.N, T = a.T;
  const int n0 = tc.a0, t0 = tc.b0;
  const int rows_n = min(G::BN, N - n0), rows_t = min(G::BT, T - t0);
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(a.Wq + (size_t)n0 * K, (uint32_t)(rows_n * K));
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(a.Xq + (size_t)t0 * K, (uint32_t)(rows_t * K));

  uint16_t bias_v = 0;  // requested before the K loop, written to LDS after it
  auto before_prologue = [&]() {
    if (a.bias && tid < G::BN && n0 + tid < N) bias_v = a.bias[n0 + tid];
    scales_to_lds<G::BN, G::BT, G::NWAVES>(a, n0, t0, rows_n, rows_t, sW_l, aX_l, wave, lane);
  };
  v16i acc[G::FN][G::FT];
  gemm_kloop<G, MmaI8>(smem, rA, rB, K, wave, lane, acc, before_prologue);
  const int fi = lane & 31, fg = lane >> 5;
  if (a.bias) {  // uniform
    if (tid < G::BN) bias_l[tid] = bias_v;
    __syncthreads();
  }

  const int nw0 = n0 + wn * G::WN, tw0 = t0 + wt * G::WT;
  const int count = *a.count;
  const int nch = (count + kOutChunk - 1) / kOutChunk;
  // Operands of the first chunk of 32 outlier columns (the common case is a
  // single chunk), all requested before the first is used so that the
  // epilogue pays one memory latency rather than one per block.
  uint4 wf0[G::FN][2], xf0[G::FT][2];
  if (nch > 0) {
#pragma unroll
    for (int i = 0; i < G::FN; ++i) {
      const int nrow = min(nw0 + i * 32 + fi, N - 1);
#pragma unroll
      for (int h = 0; h < 2; ++h)
        wf0[i][h] = *reinterpret_cast<const uint4*>(a.Wd + (size_t)nrow * kOutChunk + h * 16 + fg * 8);
    }
#pragma unroll
    for (int j = 0; j < G::FT; ++j) {
      const int t = min(tw0 + fi + j * 32, T - 1);
#pragma unroll
      for (int h = 0; h < 2; ++h)
        xf0[j][h] = *reinterpret_cast<const uint4*>(a.Xo + (size_t)t * kOutChunk + h * 16 + fg * 8);
    }
  }
  // Y through LDS in whole lines (2-slot rings only: their K loop ends with
  // every copy landed, so the whole ring is free)
  constexpr bool kCanStage = G::NSTAGE == 2 && G::FT == 2 && G::NWAVES * kStageBytes <= G::LDS;
  const bool staged = kCanStage && rows_n == G::BN && rows_t == G::BT && (N & 7) == 0;
  gemm_epilogue<BF16, G::FN, G::FT, G::BN, G::BT, G::NWAVES>(
      a, acc, wn * G::WN, wt * G::WT, sW_l + wn * G::WN, aX_l + wt * G::WT,
      a.bias ? bias_l + wn * G::WN : nullptr, count, lane, [&](int i, int h) { return wf0[i][h]; },
      [&](int j, int h) { return xf0[j][h]; },
      ChunkStaging{smem, G::LDS, wave, n0, t0, rows_n, rows_t},
      staged ? smem + wave * kStageBytes : nullptr);
}

// One wavefront column of a SplitTile: FNW row blocks from tile row wrow.
template <class G, bool BF16, int FNW>
__device__ __forceinline__ void split_column(const LinearArgs& a, char* smem, int n0, int t0, int rows_n,
                                             int rows_t, int wave, int lane, int wrow, int wcol) {
  float* sW_l = reinterpret_cast<float*>(smem + G::LDS);
  float* aX_l = sW_l + G::SW_PAD;
  uint16_t* bias_l = reinterpret_cast<uint16_t*>(aX_l + G::AX_PAD);
  const int tid = threadIdx.x;
  const int K = a.K, N = a.N;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(a.Wq + (size_t)n0 * K, (uint32_t)(rows_n * K));
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(a.Xq + (size_t)t0 * K, (uint32_t)(rows_t * K));
  uint16_t bias_v = 0;  // requested before the K loop, written to LDS after it
  auto before_prologue = [&]() {
    if (a.bias && tid < G::BN && n0 + tid < N) bias_v = a.bias[n0 + tid];
    scales_to_lds<G::BN, G::BT, G::NWAVES>(a, n0, t0, rows_n, rows_t, sW_l, aX_l, wave, lane);
  };
  const int count = *a.count;
  const int nch = (count + kOutChunk - 1) / kOutChunk;
  // The first chunk of 32 outlier columns (the common case is a single chunk):
  // the tile's BN rows of Wd and BT rows of Xo are copied into the ring slot
  // that the last K stage leaves free, while its MFMAs run (layout of
  // staged_outlier_piece).
  const char* epi = nullptr;
  auto outliers_to_lds = [&](char* free_slot) {
    epi = free_slot;
    static_assert((G::BN + G::BT) * 64 <= G::STAGE, "fits a slot");
    if (nch > 0) stage_outlier_chunk<G::BN, G::BT, G::NWAVES>(a, 0, n0, t0, rows_n, rows_t, free_slot, wave, lane);
  };
  v16i acc[FNW][G::FT];
  gemm_kloop_split<G, MmaI8, FNW>(smem, rA, rB, K, wave, lane, wrow, wcol, acc, before_prologue,
                                  outliers_to_lds);
  if (a.bias) {  // uniform
    if (tid < G::BN) bias_l[tid] = bias_v;
    __syncthreads();
  }
  const int fi = lane & 31, fg = lane >> 5;
  // Y through LDS in whole lines when the tile lies inside Y and its rows are
  // 16-byte aligned: each wavefront stages in its own part of the last slot
  static_assert(G::NWAVES * kStageBytes <= G::STAGE, "staging fits the last slot");
  const bool staged = rows_n == G::BN && rows_t == G::BT && (a.N & 7) == 0;
  char* last_slot = epi == smem ? smem + G::STAGE : smem;  // the last stage's slot, free now
  gemm_epilogue<BF16, FNW, G::FT, G::BN, G::BT, G::NWAVES>(
      a, acc, wrow, wcol, sW_l + wrow, aX_l + wcol, a.bias ? bias_l + wrow : nullptr, count,
      lane,
      [&](int i, int h) { return staged_outlier_piece(epi, wrow + i * 32 + fi, 2 * h + fg); },
      [&](int j, int h) { return staged_outlier_piece(epi, G::BN + wcol + j * 32 + fi, 2 * h + fg); },
      ChunkStaging{smem, G::LDS, wave, n0, t0, rows_n, rows_t},
      staged ? last_slot + wave * kStageBytes : nullptr);
}

template <class G, bool BF16>
__global__ __launch_bounds__(G::kThreads, 1) void kb_gemm_split(LinearArgs a, int tiles_t, int group_n) {
  __shared__ __attribute__((aligned(1024))) char smem[G::SMEM];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // wavefront column (wn) and row (wt): the two wavefronts that share a SIMD
  // (w and w + 4) take different columns, so every SIMD does the same work
  const int wn = (wave + (wave >> 2)) & 1, wt = (wave >> 1) & 3;
  const TileCoords tc = tile_coords<G>(a.N, tiles_t, group_n);
  const int n0 = tc.a0, t0 = tc.b0;
  const int rows_n = min(G::BN, a.N - n0), rows_t = min(G::BT, a.T - t0);
  if (wn == 0)
    split_column<G, BF16, G::FN0>(a, smem, n0, t0, rows_n, rows_t, wave, lane, 0, wt * G::WT);
  else
    split_column<G, BF16, G::FN1>(a, smem, n0, t0, rows_n, rows_t, wave, lane, G::FN0 * 32, wt * G::WT);
}

template <class G>
hipError_t launch_gemm_tile(const LinearArgs& a, hipStream_t stream, int group_n) {
  const int tn = (a.N + G::BN - 1) / G::BN, tt = (a.T + G::BT - 1) / G::BT;
  if (group_n < 1) group_n = 1;
  if (a.bf16)
    hipLaunchKernelGGL((kb_gemm<G, true>), dim3(tn * tt), dim3(G::kThreads), 0, stream, a, tt, group_n);
  else
    hipLaunchKernelGGL((kb_gemm<G, false>), dim3(tn * tt), dim3(G::kThreads), 0, stream, a, tt, group_n);
  return hipGetLastError();
}

template <class G>
hipError_t launch_gemm_split(const LinearArgs& a, hipStream_t stream, int group_n) {
  const int tn = (a.N + G::BN - 1) / G::BN, tt = (a.T + G::BT - 1) / G::BT;
  if (group_n < 1) group_n = 1;
  if (a.bf16)
    hipLaunchKernelGGL((kb_gemm_split<G, true>), dim3(tn * tt), dim3(G::kThreads), 0, stream, a, tt, group_n);
  else
    hipLaunchKernelGGL((kb_gemm_split<G, false>), dim3(tn * tt), dim3(G::kThreads), 0, stream, a, tt, group_n);
  return hipGetLastError();
}

// Tile shapes (BN x BT, BK, LDS stages, wavefronts along N x T).
using Tile256x256 = GemmTile<256, 256, 128, 2, 2, 4>;  // 8 wavefronts of 128x64
using Tile192x256 = GemmTile<192, 256, 128, 2, 2, 4>;  // 8 wavefronts of 96x64
using Tile256x128 = GemmTile<256, 128, 128, 2, 2, 4>;  // 8 wavefronts of 128x32
using Tile128x128 = GemmTile<128, 128, 128, 4, 2, 2>;  // 4 wavefronts of 64x64
using Tile352x256 = SplitTile<352, 256>;               // 8 wavefronts of 192x64 / 160x64

constexpr int kGroupN = 8;  // weight row-blocks per rasterization group

// Tile choice: minimise (rounds of CUs) x (time per tile), where a tile's
// time is its MFMA work divided by a per-shape efficiency (measured on gfx950:
// smaller tiles move more operand bytes per MFMA and run less efficiently; the
// 352 x 256 tile runs about as efficiently per op as 256 x 256 and exists for
// outputs that it covers in fewer rounds). `tile` >= 0 forces a candidate.
int choose_gemm_tile(int64_t T, int64_t N, int num_cus) {
  struct Cand { int bn, bt; double eff; };
  const Cand cands[kGemmTiles] = {{256, 256, 1.0}, {192, 256, 0.93}, {256, 128, 0.8}, {128, 128, 0.55},
                                  {352, 256, 1.0}};
  int best = 0;
  double best_cost = 1e300;
  for (int i = 0; i < kGemmTiles; ++i) {
    const double tiles = (double)ceil_div(N, cands[i].bn) * (double)ceil_div(T, cands[i].bt);
    const double rounds = std::ceil(tiles / num_cus);
    const double cost = rounds * cands[i].bn * cands[i].bt / cands[i].eff;
    if (cost < best_cost * 0.999) { best_cost = cost; best = i; }
  }
  return best;
}

hipError_t launch_gemm(const LinearArgs& a, int num_cus, hipStream_t stream, int tile) {
  const int best = tile >= 0 && tile < kGemmTiles ? tile : choose_gemm_tile(a.T, a.N, num_cus);
  switch (best) {
    case 0: return launch_gemm_tile<Tile256x256>(a, stream, kGroupN);
    case 1: return launch_gemm_tile<Tile192x256>(a, stream, kGroupN);
    case 2: return launch_gemm_tile<Tile256x128>(a, stream, kGroupN);
    case 3: return launch_gemm_tile<Tile128x128>(a, stream, kGroupN);
    default: return launch_gemm_split<Tile352x256>(a, stream, kGroupN);
  }
}

}  // namespace llmint8
