// Input gradient of the frozen int8 linear layer, the step that lets an
// adapter be trained on top of it ("Hugging Face Quantization with
// bitsandbytes: 4-bit & 8-bit Models Explained", the comparison table before
// section 1 and section 6: the quantized weights stay frozen while gradients
// flow through them). The stored weight is dequantized for the operation
// ("bitsandbytes" glossary, "Where it fits in the stack"):
//
//   Wdeq[n][k] = r16(fl32(fl32(Wq[n][k] * b[n]) / 127))
//   dX[t][k]   = r16( sum_n dY[t][n] * Wdeq[n][k] )  (fp32 sums)   kg_backward_dq
//
// r16 is the rounding to the 16-bit activation type: fp16, or bf16 where that
// is the compute type ("Hugging Face Quantization with bitsandbytes ...",
// section 5). kg_backward_dq forms the dequantized weight in LDS stage by
// stage from the int8 weight and multiplies on v_mfma_f32_32x32x16_{f16,bf16};
// kg_dequant_t writes the whole dequantized weight, transposed, for callers
// that want it (llmint8_dequantize_weight_t).
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
// The input gradient in one kernel, the stored weight dequantized on the fly
// for the operation ("bitsandbytes" glossary, "Where it fits in the stack"):
// no transposed copy of the weight is written.
//
//   dX[t][k] = r16( sum_n dY[t][n] * Wdeq[n][k] ),
//   Wdeq[n][k] = r16(fl32(fl32(Wq[n][k] * b[n]) * fl32(1/127)))
//
// A workgroup owns a 128 (k) x 256 (t) output tile; the reduction runs over n
// in stages of 64 (128 bytes of 16-bit operand). Stage s's dY rows sit in LDS
// slot s % 4 of B, its dequantized weight in slot s % 2 of A (160 KB in all).
// The eight wavefronts have two roles, one of each on every SIMD:
//   * four MFMA wavefronts (a 64 x 128 block each) read stage s's operands and
//     multiply on v_mfma_f32_32x32x16_{f16,bf16};
//   * four producer wavefronts fill the slots: producer p copies 64 of the
//     stage's dY rows (n contiguous) global -> LDS directly, and loads weight
//     rows n = 64 s + 16 p + r (r = 0..15), two columns per lane (the tile's
//     128 contiguous bytes of each row per instruction), with their scales,
//     both three stages ahead; one stage ahead of the MFMAs it dequantizes the
//     rows and writes, for each column, 8 consecutive n as one 16-byte piece
//     of that column's LDS row (the transposition the MFMA operand needs,
//     under the same XOR swizzle as the copied operand).
// On a SIMD the producer's VALU work thus runs beside the MFMA wavefront's
// matrix instructions with no scheduling by the compiler. Every stage ends
// with one workgroup barrier, the same number (1 + stages) in both roles.
// Each producer stage issues the same memory instructions (requests past the
// matrix use the out-of-range offset and return zero), so one vmcnt per stage
// orders them. The multiply form of the dequantization gives the division's
// result after rounding for every scale weight quantization produces (checked
// exhaustively on the host).
// ---------------------------------------------------------------------------
struct DqTile {
  static constexpr int BN = 128, BT = 256;  // output tile: k columns x t rows
  static constexpr int BK = 128;            // bytes of the reduction per stage (64 n)
  static constexpr int A_SLOTS = 2, B_SLOTS = 4;
  static constexpr int A_BYTES = BN * BK, B_BYTES = BT * BK;
  static constexpr int B_BASE = A_SLOTS * A_BYTES;  // LDS: the A slots, then the B slots
  static constexpr int LDS = B_BASE + B_SLOTS * B_BYTES;
  static constexpr int kThreads = 512;      // 4 MFMA + 4 producer wavefronts
  static constexpr int WN = 64, WT = 128;   // MFMA wavefront block
  static constexpr int FN = WN / 32, FT = WT / 32, KS = BK / 32;
  static constexpr int CPR = BK / 16, RPB = 64 / CPR;  // 16-byte chunks per row, rows per 1 KB copy
  static constexpr int B_ISSUES = BT / RPB / 4;        // 1 KB copies per producer per stage
  static constexpr int ROWS_P = 16;                    // weight rows per producer per stage
  static constexpr int LOADS = ROWS_P + 1 + B_ISSUES;  // producer memory instructions per stage
  static_assert(LDS <= 160 * 1024 && 2 * LOADS + 8 < 64, "LDS, vmcnt range");
  static_assert(4 * ROWS_P * 2 == BK && BN == 128, "4 producers x 16 rows = 64 n; 2 columns per lane");
};

// global -> LDS copy of 16 bytes per lane at voffset + soffset (soffset
// uniform); a voffset at the out-of-range offset reads zero
__device__ __forceinline__ void lds_dma16_so(__amdgpu_buffer_rsrc_t rsrc, char* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// A 16-byte LDS store the compiler does not see as a memory access. Written as
// a plain store, it would make the compiler wait, before each one, for every
// global -> LDS copy this wavefront has in flight (it cannot tell the slots
// apart), which would expose the copies' latency once per stage. These stores
// go to the A operand of a slot that no copy targets, and each stage's
// lgkmcnt(0) before the barrier orders them for the readers.
__device__ __forceinline__ void lds_store16(char* p, v4i v) {
  const uint32_t addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)p;
  asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(v));
}

template <bool BF16>
__global__ __launch_bounds__(DqTile::kThreads, 1) void kg_backward_dq(BwdArgs a, int tiles_t, int group_n) {
  using G = DqTile;
  using A16 = Act16<BF16>;
  using Mma = typename std::conditional<BF16, MmaBF16, MmaF16>::type;
  __shared__ __attribute__((aligned(1024))) char smem[G::LDS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const TileCoords tc = tile_coords<G>(a.K, tiles_t, group_n);
  const int K = a.K, N = a.N, T = a.T;
  const int Kb = 2 * N;  // reduction length in bytes of the 16-bit operands
  const int k0 = tc.a0, t0 = tc.b0;
  const int KT = (N + 63) / 64;

  if (wave >= 4) {
    // ================= producer p: weight rows 16 p .. 16 p + 15 of each stage,
    // dY rows of 1 KB blocks 4 i + p
    const int p = wave - 4;
    const int rows_k = min(G::BN, K - k0), rows_t = min(G::BT, T - t0);
    // dY rows (rows past T read as zero). Block 4 i + p is rows 8 (4 i + p) + lane / 8;
    // the lane's logical chunk is the same for every i (the swizzle depends on the
    // row mod 32), so one compare per stage finds the lanes past the reduction.
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(a.dY + (size_t)t0 * N, (uint32_t)(rows_t * Kb));
    const int pr = lane / G::CPR, pc = lane % G::CPR;
    const int kcB = (pc ^ swz<G::CPR>(p * G::RPB + pr)) * 16;
    uint32_t offB[G::B_ISSUES];
#pragma unroll
    for (int i = 0; i < G::B_ISSUES; ++i) offB[i] = (uint32_t)(((i * 4 + p) * G::RPB + pr) * Kb + kcB);
    auto issue_b = [&](int kt) {
      const int kb = kt * G::BK;
      char* sB = smem + G::B_BASE + (kt & (G::B_SLOTS - 1)) * G::B_BYTES;
      const bool in = kcB < Kb - kb;
#pragma unroll
      for (int i = 0; i < G::B_ISSUES; ++i)
        lds_dma16_so(rB, sB + (i * 4 + p) * 1024, in ? offB[i] : kOobOffset, (uint32_t)kb);
    };
    // weight rows: the windows start at the producer's first row of the stage
    // (scalar registers) and end at row N, so the per-lane offsets stay fixed;
    // rows past N and columns past the tile read as zero, and so dequantize to zero
    const bool col_ok = 2 * lane < rows_k;  // K % 16 == 0: a lane's two columns are both in or both out
    uint32_t voffW[G::ROWS_P];
#pragma unroll
    for (int r = 0; r < G::ROWS_P; ++r) voffW[r] = col_ok ? (uint32_t)(r * K + k0 + 2 * lane) : kOobOffset;
    const uint32_t voffS = (uint32_t)(lane & 15) * 4u;
    // one stage's weight words (16-bit: a 32-bit copy would make the compiler
    // zero-extend them where the loop carries them, waiting for the loads there)
    // and, in lane r of b, the scale of row r
    struct ARegs {
      uint16_t w[G::ROWS_P];
      float b;
    };
    ARegs S0, S1, S2;  // stage s in set s % 3
    auto load_a = [&](ARegs& R, int kt) {
      const int nb = kt * 64 + p * G::ROWS_P;  // uniform
      const int left = max(N - nb, 0);
      const __amdgpu_buffer_rsrc_t rW = make_rsrc(a.Wq + (size_t)min(nb, N) * K, (uint32_t)left * (uint32_t)K);
      const __amdgpu_buffer_rsrc_t rS = make_rsrc(a.sW + min(nb, N), (uint32_t)left * 4u);
#pragma unroll
      for (int r = 0; r < G::ROWS_P; ++r) R.w[r] = __builtin_amdgcn_raw_buffer_load_b16(rW, voffW[r], 0, 0);
      R.b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rS, voffS, 0, 0));
    };
    // dequantize a set and write its 4 pieces (2 columns x 2 groups of 8 rows)
    // into the A operand of stage kt's slot: column c of lane l is LDS row 2 l + c,
    // rows 8 h .. 8 h + 7 of producer p are the logical chunk 2 p + h
    auto convert_store = [&](const ARegs& R, int kt) {
      float b[G::ROWS_P];
#pragma unroll
      for (int r = 0; r < G::ROWS_P; ++r)
        b[r] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, R.b), r));
      char* sA = smem + (kt & (G::A_SLOTS - 1)) * G::A_BYTES;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int kr = 2 * lane + c;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint32_t v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r0 = 8 * h + 2 * e, r1 = r0 + 1;
            const int q0 = (int)(int8_t)(uint8_t)(R.w[r0] >> (8 * c));
            const int q1 = (int)(int8_t)(uint8_t)(R.w[r1] >> (8 * c));
            v[e] = A16::pack2(((float)q0 * b[r0]) * (1.0f / 127.0f), ((float)q1 * b[r1]) * (1.0f / 127.0f));
          }
          lds_store16(sA + kr * G::BK + (((2 * p + h) ^ swz<G::CPR>(kr)) * 16), v4i{(int)v[0], (int)v[1], (int)v[2], (int)v[3]});
        }
      }
    };
    // prologue: stages 0..2 requested (weight rows, dY rows, in that order per
    // stage; the scheduling barriers keep this order, which the wait counts),
    // stage 0's weight operand formed once its rows and dY rows have landed
    load_a(S0, 0);
    issue_b(0);
    __builtin_amdgcn_sched_barrier(0);
    load_a(S1, 1);
    issue_b(1);
    __builtin_amdgcn_sched_barrier(0);
    load_a(S2, 2);
    issue_b(2);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<2 * G::LOADS>();  // stage 0's requests have landed
    convert_store(S0, 0);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    barrier_no_fence();
    // Stage kt: on entry the MFMA wavefronts have finished stage kt - 1, so B
    // slot (kt + 3) % 4 and A slot (kt + 1) % 2 are free, and the set `load`
    // (stage kt's rows) was converted during stage kt - 1. Request stage
    // kt + 3's weight rows (into `load`) and dY rows, form stage kt + 1's
    // weight operand from `conv` (requested in stage kt - 2), then wait until
    // stage kt + 1's dY rows have landed (every request before stage kt - 1:
    // the LOADS of stages kt - 1 and kt may stay in flight) and for the LDS writes.
    auto stage = [&](int kt, const ARegs& conv, ARegs& load) {
      load_a(load, kt + 3);
      issue_b(kt + 3);
      convert_store(conv, kt + 1);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<2 * G::LOADS>();
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      barrier_no_fence();
    };
    int kt = 0;
    for (; kt + 3 <= KT; kt += 3) {
      stage(kt, S1, S0);
      stage(kt + 1, S2, S1);
      stage(kt + 2, S0, S2);
    }
    if (kt < KT) stage(kt, S1, S0);
    if (kt + 1 < KT) stage(kt + 1, S2, S1);
    wait_vmcnt<0>();  // the requests past the end (zeros into unused slots) have landed
    return;
  }

  // ================= MFMA wavefront: block (wn, wt) of the tile
  const int wn = wave & 1, wt = wave >> 1;
  const int fi = lane & 31, fg = lane >> 5;
  const int fswz = swz<G::CPR>(fi);
  int aoff[G::KS], boff[G::KS];
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks) {
    const int phys = (ks * 2 + fg) ^ fswz;
    aoff[ks] = (wn * G::WN + fi) * G::BK + phys * 16;
    boff[ks] = (wt * G::WT + fi) * G::BK + phys * 16;
  }
  typename Mma::acc_t acc[G::FN][G::FT];
#pragma unroll
  for (int i = 0; i < G::FN; ++i)
#pragma unroll
    for (int j = 0; j < G::FT; ++j) acc[i][j] = Mma::zero();
  struct Frags { v4i a[G::FN], b[G::FT]; };
  auto read_frags = [&](Frags& f, const char* sa, const char* sb, int ks) {
#pragma unroll
    for (int j = 0; j < G::FT; ++j) f.b[j] = *reinterpret_cast<const v4i*>(sb + boff[ks] + j * 32 * G::BK);
#pragma unroll
    for (int i = 0; i < G::FN; ++i) f.a[i] = *reinterpret_cast<const v4i*>(sa + aoff[ks] + i * 32 * G::BK);
  };
  auto mfma = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < G::FN; ++i)
#pragma unroll
      for (int j = 0; j < G::FT; ++j) acc[i][j] = Mma::run(f.a[i], f.b[j], acc[i][j]);
  };
  barrier_no_fence();  // the producers' prologue: stage 0's operands
  for (int kt = 0; kt < KT; ++kt) {
    const char* sa = smem + (kt & (G::A_SLOTS - 1)) * G::A_BYTES;
    const char* sb = smem + G::B_BASE + (kt & (G::B_SLOTS - 1)) * G::B_BYTES;
    Frags f0, f1;
    read_frags(f0, sa, sb, 0);
    read_frags(f1, sa, sb, 1);
    mfma(f0);
    read_frags(f0, sa, sb, 2);
    mfma(f1);
    read_frags(f1, sa, sb, 3);
    mfma(f0);
    mfma(f1);
    // one k-step of fragments ahead: each k-step's reads follow the first two
    // MFMAs of the k-step before
    constexpr int FR = G::FN + G::FT, MF = G::FN * G::FT;
    __builtin_amdgcn_sched_group_barrier(0x100, FR, 0);
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (ks + 1 < G::KS) __builtin_amdgcn_sched_group_barrier(0x100, FR, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, MF - 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    barrier_no_fence();  // the MFMAs have their operands: every read of the slots is done
  }

  // ---- epilogue: lane holds, for row t = lane&31, columns k = 8*q + 4*(lane>>5) + r
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
        uint2 pk;
        pk.x = (uint32_t)A16::from_f32(acc[i][j][4 * q]) | ((uint32_t)A16::from_f32(acc[i][j][4 * q + 1]) << 16);
        pk.y = (uint32_t)A16::from_f32(acc[i][j][4 * q + 2]) | ((uint32_t)A16::from_f32(acc[i][j][4 * q + 3]) << 16);
        *reinterpret_cast<uint2*>(a.dX + (size_t)t * K + k) = pk;
      }
    }
  }
}

hipError_t launch_backward_dq(const BwdArgs& a, int num_cus, hipStream_t stream) {
  (void)num_cus;
  using G = DqTile;
  const int tk = (a.K + G::BN - 1) / G::BN, tt = (a.T + G::BT - 1) / G::BT;
  if (a.bf16)
    hipLaunchKernelGGL(kg_backward_dq<true>, dim3(tk * tt), dim3(G::kThreads), 0, stream, a, tt, 8);
  else
    hipLaunchKernelGGL(kg_backward_dq<false>, dim3(tk * tt), dim3(G::kThreads), 0, stream, a, tt, 8);
  return hipGetLastError();
}

}  // namespace llmint8
