// Input gradient of the frozen int8 linear layer, the step that lets an
// adapter be trained on top of it ("Hugging Face Quantization with
// bitsandbytes: 4-bit & 8-bit Models Explained", the comparison table before
// section 1 and section 6: the quantized weights stay frozen while gradients
// flow through them). The stored weight is dequantized for the operation
// ("bitsandbytes" glossary, "Where it fits in the stack"):
//
//   WdT[k][n] = r16(fl32(fl32(Wq[n][k] * b[n]) / 127))           kg_dequant_t
//   dX[t][k]  = r16( sum_n dY[t][n] * WdT[k][n] )  (fp32 sums)    kg_gemm_f16
//
// r16 is the rounding to the 16-bit activation type: fp16, or bf16 where that
// is the compute type ("Hugging Face Quantization with bitsandbytes ...",
// section 5). The transposed copy makes both GEMM operands contiguous along
// the reduction (n), so the 16-bit product runs on the same direct-to-LDS K
// loop as the int8 forward (gemm_common.h) with v_mfma_f32_32x32x16_{f16,bf16}:
// a 32-byte k-step is 16 halves instead of 32 int8 values.
#include <type_traits>

#include "gemm_common.h"

namespace llmint8 {

// ---------------------------------------------------------------------------
// Dequantize + transpose. A workgroup of 256 threads owns a 64 (n) x 128 (k)
// block: it reads 64 weight rows of 128 bytes (whole cache lines), converts
// them into an LDS tile [k][n] and writes 128 rows of WdT, 128 bytes each.
// One multiply by fl32(1/127) replaces the division: for every scale that
// weight quantization produces (an fp16 or bf16 value, stored as fp32) and
// every code, the 16-bit result is the same as the division's (checked
// exhaustively on the host by the test suite; for fp16 also when the product
// is rounded to fp16 only once, as v_fma_mixlo_f16 does).
// ---------------------------------------------------------------------------
constexpr int kDqN = 64, kDqK = 128;
constexpr int kDqLd = kDqN + 2;  // halves per LDS row: 132 bytes, rows k and k+16 on different banks

template <bool BF16>
__global__ __launch_bounds__(256) void kg_dequant_t(const int8_t* __restrict__ Wq,
                                                    const float* __restrict__ sW, int N, int K,
                                                    uint16_t* __restrict__ WdT) {
  __shared__ uint16_t tile[kDqK * kDqLd];
  const int tid = threadIdx.x;
  const int n0 = blockIdx.x * kDqN, k0 = blockIdx.y * kDqK;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int e = p * 256 + tid;  // 64 rows x 8 chunks of 16 bytes
    const int r = e >> 3, c = e & 7;
    const int n = n0 + r, k = k0 + c * 16;
    if (n < N && k < K) {  // K % 16 == 0: a chunk is either whole or absent
      const uint4 v = *reinterpret_cast<const uint4*>(Wq + (size_t)n * K + k);
      const float b = sW[n];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = (int)(int8_t)((w[i >> 2] >> ((i & 3) * 8)) & 0xffu);
        tile[(c * 16 + i) * kDqLd + r] = Act16<BF16>::from_f32(((float)q * b) * (1.0f / 127.0f));
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int e = p * 256 + tid;  // 128 k-rows x 4 pieces of 16 halves
    const int kr = e >> 2, nc = (e & 3) * 16;
    const int k = k0 + kr, n = n0 + nc;
    if (k >= K || n >= N) continue;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(tile + kr * kDqLd + nc);
    uint16_t* dst = WdT + (size_t)k * N + n;
    if (n + 16 <= N) {
      uint4 lo, hi;
      lo.x = src[0]; lo.y = src[1]; lo.z = src[2]; lo.w = src[3];
      hi.x = src[4]; hi.y = src[5]; hi.z = src[6]; hi.w = src[7];
      reinterpret_cast<uint4*>(dst)[0] = lo;
      reinterpret_cast<uint4*>(dst)[1] = hi;
    } else {
      for (int i = 0; i < N - n; ++i) dst[i] = tile[kr * kDqLd + nc + i];
    }
  }
}

hipError_t launch_dequant_t(const int8_t* Wq, const float* sW, int N, int K, uint16_t* WdT,
                            bool bf16, hipStream_t stream) {
  const dim3 grid((unsigned)ceil_div(N, kDqN), (unsigned)ceil_div(K, kDqK));
  if (bf16)
    hipLaunchKernelGGL(kg_dequant_t<true>, grid, dim3(256), 0, stream, Wq, sW, N, K, WdT);
  else
    hipLaunchKernelGGL(kg_dequant_t<false>, grid, dim3(256), 0, stream, Wq, sW, N, K, WdT);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 16-bit GEMM dX = dY . WdT^T: WdT rows (output columns k) are the A operand,
// dY rows (output rows t) the B operand, both 2N bytes long.
// ---------------------------------------------------------------------------
template <class G, bool BF16>
__global__ __launch_bounds__(G::kThreads, 1) void kg_gemm_f16(BwdArgs a, int tiles_t, int group_n) {
  using A16 = Act16<BF16>;
  using Mma = typename std::conditional<BF16, MmaBF16, MmaF16>::type;
  __shared__ __attribute__((aligned(1024))) char smem[G::LDS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % G::WAVES_N, wt = wave / G::WAVES_N;

  const TileCoords tc = tile_coords<G>(a.K, tiles_t, group_n);
  const int K = a.K, N = a.N, T = a.T;
  const int Kb = 2 * N;  // reduction length in bytes
  const int k0 = tc.a0, t0 = tc.b0;
  const int rows_k = min(G::BN, K - k0), rows_t = min(G::BT, T - t0);
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(a.WdT + (size_t)k0 * N, (uint32_t)(rows_k * Kb));
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(a.dY + (size_t)t0 * N, (uint32_t)(rows_t * Kb));

  v16f acc[G::FN][G::FT];
  gemm_kloop<G, Mma>(smem, rA, rB, Kb, wave, lane, acc, [] {});

  // Output block layout: lane holds, for row t = lane&31, columns
  // k = 8*q + 4*(lane>>5) + r in register 4*q + r (q, r = 0..3).
  const int fi = lane & 31, fg = lane >> 5;
  const int kl = k0 + wn * G::WN + 4 * fg;
  const int tl = t0 + wt * G::WT + fi;
#pragma unroll
  for (int i = 0; i < G::FN; ++i) {
#pragma unroll
    for (int j = 0; j < G::FT; ++j) {
      const int t = tl + j * 32;
      if (t >= T) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = kl + i * 32 + 8 * q;
        if (k >= K) continue;  // K % 16 == 0: the 4 columns are all in range
        uint2 p;
        p.x = (uint32_t)A16::from_f32(acc[i][j][4 * q]) |
              ((uint32_t)A16::from_f32(acc[i][j][4 * q + 1]) << 16);
        p.y = (uint32_t)A16::from_f32(acc[i][j][4 * q + 2]) |
              ((uint32_t)A16::from_f32(acc[i][j][4 * q + 3]) << 16);
        *reinterpret_cast<uint2*>(a.dX + (size_t)t * K + k) = p;
      }
    }
  }
}

template <class G>
hipError_t launch_gemm_f16_tile(const BwdArgs& a, hipStream_t stream, int group_n) {
  const int tk = (a.K + G::BN - 1) / G::BN, tt = (a.T + G::BT - 1) / G::BT;
  if (a.bf16)
    hipLaunchKernelGGL((kg_gemm_f16<G, true>), dim3(tk * tt), dim3(G::kThreads), 0, stream, a, tt, group_n);
  else
    hipLaunchKernelGGL((kg_gemm_f16<G, false>), dim3(tk * tt), dim3(G::kThreads), 0, stream, a, tt, group_n);
  return hipGetLastError();
}

using BTile256x256 = GemmTile<256, 256, 128, 2, 2, 4>;  // 8 wavefronts of 128x64
using BTile256x128 = GemmTile<256, 128, 128, 2, 4, 2>;  // 8 wavefronts of 64x64
using BTile128x256 = GemmTile<128, 256, 128, 2, 2, 4>;  // 8 wavefronts of 64x64
using BTile128x128 = GemmTile<128, 128, 128, 4, 2, 2>;  // 4 wavefronts of 64x64

hipError_t launch_gemm_f16_variant(const BwdArgs& a, int variant, hipStream_t stream) {
  switch (variant) {
    case 0: return launch_gemm_f16_tile<BTile256x256>(a, stream, 8);
    case 1: return launch_gemm_f16_tile<BTile256x128>(a, stream, 8);
    case 2: return launch_gemm_f16_tile<BTile128x256>(a, stream, 8);
    default: return launch_gemm_f16_tile<BTile128x128>(a, stream, 8);
  }
}

// Tile choice: fewest rounds of CUs, then the larger tile (fewer operand bytes
// per MFMA).
hipError_t launch_gemm_f16(const BwdArgs& a, int num_cus, hipStream_t stream) {
  struct Cand { int bk, bt, variant; };
  const Cand cands[] = {{256, 256, 0}, {256, 128, 1}, {128, 256, 2}, {128, 128, 3}};
  int best = 0;
  double best_cost = 1e300;
  for (int i = 0; i < 4; ++i) {
    const double tiles = (double)ceil_div(a.K, cands[i].bk) * (double)ceil_div(a.T, cands[i].bt);
    const double rounds = std::ceil(tiles / num_cus);
    // time per round ~ tile area; smaller tiles move more bytes per MFMA
    const double eff = i == 0 ? 1.0 : (i < 3 ? 0.8 : 0.55);
    const double cost = rounds * cands[i].bk * cands[i].bt / eff;
    if (cost < best_cost * 0.999) { best_cost = cost; best = i; }
  }
  return launch_gemm_f16_variant(a, cands[best].variant, stream);
}

}  // namespace llmint8
