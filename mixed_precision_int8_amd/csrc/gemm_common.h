// K-loops shared by the gfx950 GEMM kernels of this library: tile shapes,
// the direct-to-LDS copy ring and the MFMA software pipeline. A kernel supplies
// the two operands as K-contiguous byte rows (A: BN rows, B: BT rows), the MFMA
// flavour, and its own epilogue; the loop leaves each wavefront's accumulators
// in registers as 32x32 blocks. gemm_kloop serves evenly split tiles
// (GemmTile: (BN/WAVES_N) x (BT/WAVES_T) per wavefront, fragments
// double-buffered); gemm_kloop_split serves SplitTile, whose two wavefront
// columns may differ by one row block and whose accumulators leave room for a
// single set of fragment registers only.
//
// Design (CDNA4): K-stages of BK bytes are copied global->LDS with
// buffer_load_dwordx4 ... lds (no VGPR staging) into a ring of NSTAGE buffers,
// NSTAGE-1 stages in flight; rows and K beyond the matrix read as zero through
// the buffer range check. The ring is synchronised with partial vmcnt waits
// and a fence-free s_barrier, so the prefetch is never drained. LDS rows carry
// an XOR swizzle of their 16-byte chunks chosen so that the fragment reads
// (ds_read_b128) are bank-conflict free. Blocks are remapped so that each XCD
// (own L2) works on a contiguous range of tiles sharing operand panels.
#pragma once

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


// MFMA flavours: one 32x32 output block per call, operands are 16 bytes per lane
// of a 32-byte k-step (32 int8 values, or 16 fp16 values).
struct MmaI8 {
  typedef v16i acc_t;
  static __device__ __forceinline__ acc_t zero() {
    acc_t z;
#pragma unroll
    for (int v = 0; v < 16; ++v) z[v] = 0;
    return z;
  }
  static __device__ __forceinline__ acc_t run(v4i a, v4i b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
  }
};
struct MmaF16 {
  typedef v16f acc_t;
  static __device__ __forceinline__ acc_t zero() {
    acc_t z;
#pragma unroll
    for (int v = 0; v < 16; ++v) z[v] = 0.0f;
    return z;
  }
  static __device__ __forceinline__ acc_t run(v4i a, v4i b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a),
                                                   __builtin_bit_cast(v8h, b), c, 0, 0, 0);
  }
};

struct MmaBF16 {
  typedef v16f acc_t;
  static __device__ __forceinline__ acc_t zero() { return MmaF16::zero(); }
  static __device__ __forceinline__ acc_t run(v4i a, v4i b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a),
                                                    __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
  }
};

// Tile order. Hardware deals blocks round-robin over the 8 XCDs; each XCD gets
// a contiguous run of tile ids. Ids are then grouped: group_n A row-blocks
// sweep all B row-blocks with A fastest, so the tiles an XCD runs concurrently
// share a few operand panels and most K-slices are hits in that XCD's L2.
struct TileCoords {
  int a0, b0;  // first A row (output column) and first B row (output row)
};
template <class G>
__device__ __forceinline__ TileCoords tile_coords(int rows_a, int tiles_b, int group_n) {
  const int nb = gridDim.x, b = blockIdx.x;
  const int nb8 = nb & ~7;
  const int id = b < nb8 ? (b & 7) * (nb8 >> 3) + (b >> 3) : b;
  const int tiles_a = (rows_a + G::BN - 1) / G::BN;
  const int per_group = group_n * tiles_b;
  const int grp = id / per_group, in_grp = id % per_group;
  const int gn = min(group_n, tiles_a - grp * group_n);
  TileCoords c;
  c.a0 = (grp * group_n + in_grp % gn) * G::BN;
  c.b0 = (in_grp / gn) * G::BT;
  return c;
}

// The K loop. rA / rB cover the tile's A and B rows (Kb bytes each, K-contiguous);
// `before_prologue` runs just before the first copies are issued (a kernel
// issues extra direct copies of its own there: the stage waits cover them).
template <class G, class Mma, class Pre>
__device__ __forceinline__ void gemm_kloop(char* smem, __amdgpu_buffer_rsrc_t rA,
                                           __amdgpu_buffer_rsrc_t rB, int Kb, int wave, int lane,
                                           typename Mma::acc_t (&acc)[G::FN][G::FT],
                                           Pre&& before_prologue) {
  const int wn = wave % G::WAVES_N, wt = wave / G::WAVES_N;
  const int K = Kb;
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

#pragma unroll
  for (int i = 0; i < G::FN; ++i)
#pragma unroll
    for (int j = 0; j < G::FT; ++j) acc[i][j] = Mma::zero();
  auto mfma = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < G::FN; ++i)
#pragma unroll
      for (int j = 0; j < G::FT; ++j)
        acc[i][j] = Mma::run(f.a[i], f.b[j], acc[i][j]);
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
  before_prologue();
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
}

// Tiles whose accumulators take most of a wavefront's registers: 8
// wavefronts, 2 along N x 4 along T, 2-slot ring of 128-byte stages. BN need
// not split evenly: the wavefront columns own ceil(BN/64) and floor(BN/64)
// 32-row blocks (352 = 192 + 160 rows), and the copy of A is spread over the
// wavefronts as evenly as 1 KB pieces allow. With 2 slots every stage waits
// for all of its copies (vmcnt(0)), so the per-wavefront copy counts may differ.
template <int BN_, int BT_>
struct SplitTile {
  static constexpr int BN = BN_, BT = BT_, BK = 128, NSTAGE = 2;
  static constexpr int WAVES_T = 4, NWAVES = 8, kThreads = 64 * NWAVES;
  static constexpr int NB = BN / 32;                       // 32-row blocks along N
  static constexpr int FN0 = (NB + 1) / 2, FN1 = NB - FN0;  // per wavefront column
  static constexpr int WT = BT / WAVES_T, FT = WT / 32;
  static constexpr int KS = BK / 32, CPR = BK / 16, RPB = 64 / CPR;
  static constexpr int A_BYTES = BN * BK, B_BYTES = BT * BK, STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS = STAGE * NSTAGE;
  static constexpr int A_BLOCKS = BN / RPB;                 // 1 KB copy pieces of A per stage
  static constexpr int A_ISSUES = (A_BLOCKS + NWAVES - 1) / NWAVES, A_FULL = A_BLOCKS / NWAVES;
  static constexpr int B_ISSUES = BT / RPB / NWAVES;
  // scales are copied in 64-entry pieces; the arrays are padded to whole pieces
  static constexpr int SW_PAD = (BN + 63) / 64 * 64, AX_PAD = (BT + 63) / 64 * 64;
  static constexpr int SMEM = LDS + (SW_PAD + AX_PAD) * 4 + BN * 2;
  static_assert(BN % 32 == 0 && FT == 2 && BT % (RPB * NWAVES) == 0, "tile shape");
  static_assert((NWAVES * RPB) % 32 == 0, "copy pieces keep the row swizzle");
  static_assert(BN <= kThreads && SMEM <= 160 * 1024, "LDS");
};

// K loop of a SplitTile wavefront owning FNW x FT accumulator blocks, A rows
// wrow.. and B rows wcol.. of the tile. The fragments are single-buffered:
// MFMAs run column-block major (all i for j = 0, then all i for j = 1) and each
// fragment is replaced by the next k-step's right after its last use, which
// gives every read about FNW MFMAs of lead and leaves the registers to the
// accumulators. The last stage has no successor to copy: `into_free_slot`
// receives the ring slot it leaves free and may fill it with direct copies
// (covered by that stage's wait and barrier).
template <class G, class Mma, int FNW, class Pre, class Last>
__device__ __forceinline__ void gemm_kloop_split(char* smem, __amdgpu_buffer_rsrc_t rA,
                                                 __amdgpu_buffer_rsrc_t rB, int K, int wave, int lane,
                                                 int wrow, int wcol,
                                                 typename Mma::acc_t (&acc)[FNW][G::FT],
                                                 Pre&& before_prologue, Last&& into_free_slot) {
  constexpr int FT = G::FT;
  // Copy piece i of a wavefront holds rows (i * NWAVES + wave) * RPB + lane / CPR;
  // i * NWAVES * RPB is a multiple of 32, so every piece has the same swizzled
  // chunk and the offsets step by the uniform NWAVES * RPB * K.
  const int pr = lane / G::CPR, pc = lane % G::CPR;
  const int row0 = wave * G::RPB + pr;
  const int kc = (pc ^ swz<G::CPR>(row0)) * 16;
  const uint32_t off0 = (uint32_t)(row0 * K + kc);
  const uint32_t istride = (uint32_t)(G::NWAVES * G::RPB * K);
  auto issue = [&](int slot, int kt) {
    const int kb = kt * G::BK;
    char* sA = smem + slot * G::STAGE;
    char* sB = sA + G::A_BYTES;
    const bool ok = kb + G::BK <= K || kb + kc < K;  // K past the end reads zeros
    const uint32_t o = off0 + kb;
#pragma unroll
    for (int i = 0; i < G::A_ISSUES; ++i)
      if (i < G::A_FULL || i * G::NWAVES + wave < G::A_BLOCKS)
        lds_dma16(rA, sA + (i * G::NWAVES + wave) * 1024, ok ? o + i * istride : kOobOffset);
#pragma unroll
    for (int i = 0; i < G::B_ISSUES; ++i)
      lds_dma16(rB, sB + (i * G::NWAVES + wave) * 1024, ok ? o + i * istride : kOobOffset);
  };
  // fragment addresses: the per-lane part (row fi, swizzled chunk of k-step ks)
  // is the same for A and B
  const int fi = lane & 31, fg = lane >> 5;
  const int fswz = swz<G::CPR>(fi);
  int loff[G::KS];
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks) loff[ks] = fi * G::BK + ((ks * 2 + fg) ^ fswz) * 16;
  const int abase = wrow * G::BK, bbase = G::A_BYTES + wcol * G::BK;
  v4i fa[FNW], fb[FT];
  auto read_a = [&](int i, int slot, int ks) {
    fa[i] = *reinterpret_cast<const v4i*>(smem + slot * G::STAGE + abase + loff[ks] + i * 32 * G::BK);
  };
  auto read_b = [&](int j, int slot, int ks) {
    fb[j] = *reinterpret_cast<const v4i*>(smem + slot * G::STAGE + bbase + loff[ks] + j * 32 * G::BK);
  };
#pragma unroll
  for (int i = 0; i < FNW; ++i)
#pragma unroll
    for (int j = 0; j < FT; ++j) acc[i][j] = Mma::zero();
  // MFMAs of the fragments in registers; each fragment then receives k-step
  // (nslot, nks)
  auto step = [&](int nslot, int nks) {
#pragma unroll
    for (int i = 0; i < FNW; ++i) acc[i][0] = Mma::run(fa[i], fb[0], acc[i][0]);
    read_b(0, nslot, nks);
#pragma unroll
    for (int i = 0; i < FNW; ++i) {
      acc[i][1] = Mma::run(fa[i], fb[1], acc[i][1]);
      read_a(i, nslot, nks);
    }
    read_b(1, nslot, nks);
    __builtin_amdgcn_sched_group_barrier(0x008, FNW, 0);  // MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // DS read
#pragma unroll
    for (int i = 0; i < FNW; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  };
  const int KT = (K + G::BK - 1) / G::BK;
  // stage kt in `slot`: copy the next stage (or hand over the free slot), the
  // MFMAs of k-steps 0..KS-2 with the reads of 1..KS-1, then the waits and the
  // barrier; the MFMAs of its last k-step run after the barrier, with the reads
  // of the next stage's first.
  auto body = [&](int slot, int kt) {
    if (kt + 1 < KT) issue(slot ^ 1, kt + 1);
    else into_free_slot(smem + (slot ^ 1) * G::STAGE);
#pragma unroll
    for (int ks = 1; ks < G::KS; ++ks) step(slot, ks);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    barrier_no_fence();
  };
  before_prologue();
  issue(0, 0);
  wait_vmcnt<0>();
  barrier_no_fence();
#pragma unroll
  for (int i = 0; i < FNW; ++i) read_a(i, 0, 0);
#pragma unroll
  for (int j = 0; j < FT; ++j) read_b(j, 0, 0);
  body(0, 0);
  int slot = 1;
  for (int kt = 1; kt < KT; ++kt) {
    step(slot, 0);
    body(slot, kt);
    slot ^= 1;
  }
#pragma unroll
  for (int j = 0; j < FT; ++j)
#pragma unroll
    for (int i = 0; i < FNW; ++i) acc[i][j] = Mma::run(fa[i], fb[j], acc[i][j]);
}

// Output staging for the GEMM epilogues. A wavefront's results for a pair of
// 32-row blocks (i even, i + 1) and its 64 output rows are gathered in a
// private LDS area as 64 rows of 128 bytes, then stored as whole 128-byte
// lines (8 rows per instruction) instead of 16-byte pieces of 32 rows.
constexpr int kStagePitch = 144;  // bytes per staged row: 128 + 16 (conflict-free writes)
constexpr int kStageBytes = 64 * kStagePitch;

// the 4 packed 16-bit values (columns 8q + 4fg .. +3 of block i, output row
// 32j + fi) of one lane
__device__ __forceinline__ void stage_put(char* stage, int i, int j, int q, int fi, int fg, uint2 p) {
  *reinterpret_cast<uint2*>(stage + (j * 32 + fi) * kStagePitch + (i & 1) * 64 + 8 * fg + 16 * q) = p;
}

// the staged nb (1 or 2) blocks -> out[row * ld + 0 .. nb * 32), rows 0..63.
// The stores are non-temporal: Y is not read again by the kernel, and its lines
// then go to memory without taking L2 space from the operand panels (same
// bits; 347 against 373 us at the 2048 x 14336 x 14336 layer, 748 against 760 us
// at 4096 x 8192 x 28672, unchanged at 2048 x 4096 x 11008, where every tile
// stores at the end at once)
__device__ __forceinline__ void stage_flush(const char* stage, int nb, int lane, uint16_t* out, size_t ld) {
  const int cpr = 4 * nb, rpp = 64 / cpr;  // 16-byte chunks per row, rows per pass
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k * rpp >= 64) break;
    const int row = lane / cpr + k * rpp, c = lane % cpr;
    const uint4 v = *reinterpret_cast<const uint4*>(stage + row * kStagePitch + c * 16);
    __builtin_nontemporal_store(__builtin_bit_cast(v4i, v), reinterpret_cast<v4i*>(out + (size_t)row * ld + c * 8));
  }
}

}  // namespace llmint8
