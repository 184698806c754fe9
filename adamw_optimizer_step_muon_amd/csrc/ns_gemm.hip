// Newton-Schulz matrix products on the gfx950 matrix cores (bf16 in, fp32 accumulate).
//
// One iteration of the quintic ("Optimizers: AdamW, Muon and the distributed
// optimizer", section "Muon: orthogonalising the update", newton_schulz listing) on
// an m x n bf16 matrix X (m <= n):
//
//   gram:     R  = X X^T                  m x m, symmetric
//   poly:     P  = a I + b R + c R R^T    m x m, symmetric (R R^T = R^2 as R = R^T)
//   combine:  X' = P X                    m x n
//
// a X + (b R + c R^2) X = (a I + b R + c R^2) X, so the a X term rides on P's
// diagonal: P is formed in fp32 and rounded to bf16 once, and the combine is a plain
// product with no second read of X in its epilogue.
//
// The Gram and polynomial products are C = A B^T with both operands stored row-major
// along the contraction index, the layout of the MFMA operands:
//   gram     A = B = X  (contraction over n)
//   poly     A = B = R  (contraction over m)
// The combine is C = A B with B = X stored row-major along n: its LDS stage holds k
// rows of X and the B fragments are read with gfx950's transposing LDS load
// (ds_read_b64_tr_b16), so X is kept in one orientation only; for Gram sides above
// 2048 it reads a stored X^T instead (C = A B^T like the others):
//   combine  A = P, B = X or X^T (contraction over m)
// Symmetric outputs are computed on lower-triangle tiles only and mirrored, halving
// the work of the two symmetric products ("DMuon: Efficient Distributed Muon Training
// with Near-Adam Overhead", section 2.2, symmetry exploitation); same-shape matrices
// are batched in one launch (same section, batching).
//
// Kernel structure (one template, 256 x 256 and 128 x 128 tiles):
//   * BM x BN output tile per block, WM x WN waves, v_mfma_f32_32x32x16_bf16;
//   * operands stream HBM/L2 -> LDS with buffer_load_dwordx4 ... lds (no register
//     staging) into rings of SA stages of A and SB of B; each 16-byte chunk of an
//     operand row is XOR-swizzled so the 32 rows one MFMA fragment reads fall on
//     distinct banks;
//     the swizzle is applied on the global side, since LDS-DMA writes each wave's
//     64 chunks contiguously;
//   * blocks are renumbered (they go round-robin to the 8 XCDs): for matrices of a
//     few hundred tiles or fewer each XCD works on a contiguous run of tiles, grouped
//     by row panels, so the blocks resident on one XCD share operand panels in its L2;
//     larger matrices are shared by the eight XCDs, so the panels one XCD's L2 misses
//     are likely in the memory-side cache from another;
//   * epilogue: b/c terms (and a on the diagonal) or the first iteration's
//     normalisation in fp32 in registers, round to bf16; the tile is staged once in an
//     XOR-swizzled LDS tile and both orientations (row-major, and the transposed /
//     mirrored copy) leave with 16-byte row stores, the second through transposing
//     LDS reads.
// Sizes are padded to the tile by the caller and the padding is zero (preserved by
// the iteration), so there are no bounds checks inside.
#include <cstdlib>
#include <type_traits>

#include "ma_internal.h"

typedef int i32x4 __attribute__((ext_vector_type(4)));
// buffer_load_dwordx4 ... lds: 16 bytes per lane from a buffer resource into LDS, the
// wave's 64 chunks contiguous from LDS byte address m0.  Measured faster than the
// global form (global_load_lds_dwordx4) by 2-6 % on 8192-wide and 13 % on 768-wide
// Gram products.  Declared at file scope: the name binds to the LLVM intrinsic.
__device__ void raw_buffer_load_lds(i32x4 rsrc, __attribute__((address_space(3))) unsigned* lds,
                                    int size, int voffset, int soffset, int offset,
                                    int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

namespace ma {
namespace {

template <int BM_, int BN_, int BK_, int WM_, int WN_, int STAGES_, bool READS_X_,
          int BSTAGES_ = STAGES_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, STAGES = STAGES_;
  // ring depths of the A and B operand stages: equal, or 3 and 2 (either way round),
  // the deeper operand being loaded one stage further ahead
  static constexpr int SA = STAGES_, SB = BSTAGES_;
  static constexpr int LA = SA - 1, LB = SB - 1;  // stages loaded ahead
  static constexpr int kLead = LA > LB ? LA : LB;
  static_assert(SB == SA || (SB == SA + 1 && SA == 2) || (SA == SB + 1 && SB == 2),
                "ring depths");
  // in each issue group the operand with the shorter lead goes first
  static constexpr bool kBFirst = SA > SB;
  // combine operand B: X itself through transposing LDS reads (true), or the stored
  // transpose X^T through plain b128 reads (false)
  static constexpr bool kCombineReadsX = READS_X_;
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int WTM = BM / (WM * 32);  // 32x32 MFMA tiles per wave along M
  static constexpr int WTN = BN / (WN * 32);
  static constexpr int kChunks = BK / 8;              // 16-byte chunks per operand row
  static constexpr int kRowsPerDma = 64 / kChunks;    // rows one wave-wide LDS-DMA fills
  static constexpr int kDmaA = BM / kRowsPerDma / kWaves;  // per wave per stage
  static constexpr int kDmaB = BN / kRowsPerDma / kWaves;
  static constexpr int kDmaPerStage = kDmaA + kDmaB;
  static constexpr int kAElems = BM * BK, kBElems = BN * BK;  // one stage of A / of B
  static constexpr int kBBase = SA * kAElems;                   // B ring after the A ring
  static constexpr int kMainElems = SA * kAElems + SB * kBElems;
  static constexpr int kEpiElems = BM * BN;
  static constexpr int kLdsElems = kMainElems > kEpiElems ? kMainElems : kEpiElems;
  // Take the polynomial's b R term from the B operand stage that covers the tile's
  // rows (R[i][j] = R[j][i]) instead of reading it again from memory; held in
  // registers, so only where the wave tile is small.
  static constexpr bool kCaptureAux = (WTM * WTN) <= 4;
  static_assert(BM % (WM * 32) == 0 && BN % (WN * 32) == 0, "wave tiling");
  static_assert(BM % (kRowsPerDma * kWaves) == 0 && BN % (kRowsPerDma * kWaves) == 0, "dma");
  static_assert(BK == 32 || BK == 64, "swizzle defined for BK 32 and 64");
  static_assert(kLdsElems * 2 <= 160 * 1024, "LDS");
};

// 16-byte chunk swizzle inside an operand row (an involution in c).  A fragment read
// has 32 lanes on 32 consecutive rows at one logical chunk (the other half-wave on the
// next chunk).  Both masks were measured free of bank conflicts for that read on gfx950
// (ds_read_b128 throughput at 16 waves per CU equal to the best pattern; the 64-byte
// row mask ((r >> 1) ^ (r >> 3)) & 3, which also looks conflict-free on a plain 64-bank
// model, measured 2-way).
template <int BK>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (BK == 64) return c ^ ((r ^ (r >> 3)) & 7);         // 8 chunks per row
  else return c ^ ((r ^ (r >> 2)) & 3);                            // 4 chunks per row
}

// 16-byte chunk swizzle of a k row of the combine's B stage ([BK][BN], n contiguous):
// the transposing reads of one instruction cover 4 consecutive k rows of 64 bytes per
// 16-lane group; XOR-ing the chunk with 4 (r % 4) puts those rows on distinct banks
// (measured conflict-free on gfx950, like (r % 8) combined with higher row bits; with
// no swizzle the read runs at about a third of the rate).
__device__ __forceinline__ int swz_kn(int r, int c) { return c ^ ((r & 3) << 2); }

// 16-byte chunk c of row j of a transposed epilogue tile with N chunks per row: XOR with
// j for power-of-two N, a rotation by j otherwise (the 24 chunks of 192-row tiles); a
// permutation of the row's chunks either way.
template <int N>
__device__ __forceinline__ int tswz(int c, int j) {
  if constexpr ((N & (N - 1)) == 0) return c ^ (j % N);
  else return (c + j) % N;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// One 32 x 32 x 16 MFMA on 16-bit operands (kTy: GemmTypes): bf16, or fp16 (the
// Gram-space products; same rate).  The fragments are loaded as raw 16-bit values.
template <int kTy>
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (kTy == kTyBf16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}
// fp32 result -> the 16-bit type a launch writes, and a 16-bit operand -> fp32.  The
// fp16 conversion takes the finished fp32 value: the compiler would otherwise fold it
// into the epilogue's last multiply-add (v_fma_mixlo_f16, one rounding instead of two)
// in some instantiations and not in others, so tile shapes would differ in the last
// bit (the empty asm only pins the value in a register; it emits nothing).
template <int kTy>
__device__ __forceinline__ unsigned short to16(float f) {
  if constexpr (kTy == kTyF16) {
    asm volatile("" : "+v"(f));
    return f2h(f);
  } else {
    return f2bf(f);
  }
}
template <int kTy>
__device__ __forceinline__ float from16(unsigned short h) {
  if constexpr (kTy == kTyBf16) return bf2f(h);
  else return h2f(h);
}

// 4 bf16 of a column block: lane i of each 16-lane group receives element i % 4 of the
// 8 bytes addressed by lane 4 e + i / 4 of its group, as element e (e = 0..3).
__device__ __forceinline__ s16x4 lds_read_tr(const unsigned short* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// wait until at most n vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// The block-wide step between two operand stages: this wave's LDS reads have completed
// (lgkmcnt(0)), then s_barrier.  After it other waves load the next stages into the
// slots just read, so no read of those slots may be left behind it.  The s_barrier
// builtin does not order memory accesses for the compiler: in the polynomial kernels
// with 128-row tiles it moved a stage's last fragment reads (whose only uses, the
// stage's last MFMAs, follow the barrier) into the block after it, and the results
// changed from run to run.  As one asm statement with a memory clobber neither the
// reads nor the DMAs can cross it.  The builtin lgkmcnt(0) before it is the same wait,
// visible to the compiler's own wait counting.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0), vmcnt and expcnt untouched
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}


// Resource of a buffer of `bytes` bytes at the wave-uniform `base` (reads past `bytes`
// return zero: the hardware range check).
__device__ __forceinline__ i32x4 buffer_rsrc(const unsigned short* base, unsigned bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(a & 0xffffffffu));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>(a >> 32));  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));     // num_records
  r[3] = 0x00020000;  // gfx9 raw buffer: 32-bit data format, no swizzle
  return r;
}

// 16-byte load at byte offset voff (per lane) of that buffer into LDS at l.
//
// kAsm: issued as inline assembly.  The compiler's wait-count pass treats an LDS DMA
// it knows about as a write that may alias any later LDS read carrying a memory
// operand (ds_read_b64_tr_b16 does; the plain fragment reads do not), and put an
// s_waitcnt vmcnt(0) before every transposing read -- each stage then waited for the
// next stage's DMA.  The kernel orders DMA and reads itself (wait_vmcnt on its own
// stage, then s_barrier).  Only the kernels with transposing reads use it: elsewhere
// the intrinsic schedules better (the asm's memory clobber measured 3 % slower on the
// 256-tile kernels that read X^T).
template <bool kAsm>
__device__ __forceinline__ void dma16(const unsigned short* base, int voff, unsigned bytes,
                                      unsigned short* l) {
  const i32x4 r = buffer_rsrc(base, bytes);
  if constexpr (kAsm) {
    const int lds = __builtin_amdgcn_readfirstlane(static_cast<int>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned short*)(l))));
    // m0 (the LDS address) is an input operand: the compiler sets it and knows its value
    asm volatile(
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, 0 offen lds"
        :
        : "v"(voff), "s"(r), "{m0}"(lds)
        : "memory");
  } else {
    raw_buffer_load_lds(r, (__attribute__((address_space(3))) unsigned*)(l), 16, voff, 0, 0, 0);
  }
}

template <class C, int kEpi, int kTy = kTyBf16>
__global__ __launch_bounds__(C::kThreads) void ns_gemm_kernel(GemmTable table) {
  __shared__ __attribute__((aligned(16))) unsigned short smem[C::kLdsElems];
  // The table is read in place from the kernel-argument segment with the (uniform)
  // group index (the compiler turns these into scalar loads), not copied privately.
  const GemmTable* kt = (const GemmTable*)__builtin_amdgcn_kernarg_segment_ptr();
  (void)table;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the wave index is uniform across the wave: as a scalar it keeps the per-wave LDS
  // destinations of the operand DMAs (the m0 operand) and the fragment bases in scalar
  // registers, which halved the main loop's vector ALU instructions (76 -> 38 per
  // stage of the 256-tile kernels) and measured 0.4 % faster on 8192-wide Gram sides
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN;
  const int wn = wave % C::WN;

  // block -> (group, matrix, tile row, tile column): the same function the host-side
  // plan check enumerates; padding blocks exit at once
  int gi, ti, tj;
  int64_t batch;
  if (!gemm_block_tile(*kt, kEpi, static_cast<int>(blockIdx.x), gi, batch, ti, tj)) return;
  const GemmArgs args = kt->g[gi];
  const int64_t m0 = static_cast<int64_t>(ti) * C::BM;
  const int64_t n0 = static_cast<int64_t>(tj) * C::BN;

  // combine reading X: B is staged as k rows of BN columns starting at column n0
  constexpr bool kBT = (kEpi == kCombine) && C::kCombineReadsX;
  const unsigned short* gA = args.A + batch * args.strideA + m0 * args.lda;
  const unsigned short* gB = args.B + batch * args.strideB + (kBT ? n0 : n0 * args.ldb);

  const int nk = args.kdim / C::BK;
  // LDS-DMA source pointers for this lane (k offset added per stage)
  const int drow = lane / C::kChunks;  // row inside one DMA
  const int dpc = lane % C::kChunks;   // physical chunk this lane fills
  // DMA number d of one issue group of this wave: the operand with the shorter lead
  // first (A when the rings are equal), then the other
  auto is_a = [](int d) { return C::kBFirst ? d >= C::kDmaB : d < C::kDmaA; };
  auto issue_one = [&](int kt, int d) {
    unsigned short* as = smem + (kt % C::SA) * C::kAElems;
    unsigned short* bs = smem + C::kBBase + (kt % C::SB) * C::kBElems;
    const int k0 = kt * C::BK;
    const bool isA = is_a(d);
    const int i = C::kBFirst ? (isA ? d - C::kDmaB : d) : (isA ? d : d - C::kDmaA);
    const int r0 = (i * C::kWaves + wave) * C::kRowsPerDma;
    const int r = r0 + drow;
    // one buffer per operand stage, based at its first element; offsets and extents
    // stay below 2^30 bytes (sides are at most 2^20)
    const int lda = static_cast<int>(args.lda), ldb = static_cast<int>(args.ldb);
    if (isA) {
      dma16<kBT>(gA + k0, (r * lda + swz<C::BK>(r, dpc) * 8) * 2,
                 static_cast<unsigned>(((C::BM - 1) * lda + C::BK) * 2), as + r0 * C::BK);
    } else if constexpr (kBT) {
      // [BK][BN] stage: one DMA fills kBRows k rows of BN columns (1 KiB)
      constexpr int kBChunks = C::BN / 8, kBRows = 64 / kBChunks;
      const int q0 = (i * C::kWaves + wave) * kBRows;
      const int q = q0 + lane / kBChunks, pc = lane % kBChunks;
      dma16<kBT>(gB + static_cast<int64_t>(k0) * args.ldb, (q * ldb + swz_kn(q, pc) * 8) * 2,
                 static_cast<unsigned>(((C::BK - 1) * ldb + C::BN) * 2), bs + q0 * C::BN);
    } else {
      dma16<kBT>(gB + k0, (r * ldb + swz<C::BK>(r, dpc) * 8) * 2,
                 static_cast<unsigned>(((C::BN - 1) * ldb + C::BK) * 2), bs + r0 * C::BK);
    }
  };
  // DMA d of issue group v: A of stage v + LA when is_a(d), else B of stage v + LB.
  // Group v goes out at the start of stage v, after the barrier that ended stage v - 1,
  // into the slots that stage v - 1 read; the prologue issues groups -kLead .. -1.
  auto issue_group_one = [&](int v, int d) {
    const int st = v + (is_a(d) ? C::LA : C::LB);
    if (st >= 0 && st < nk) issue_one(st, d);
  };

  f32x16 acc[C::WTM][C::WTN];
#pragma unroll
  for (int i = 0; i < C::WTM; ++i)
#pragma unroll
    for (int j = 0; j < C::WTN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  constexpr int KK = C::BK / 16;  // MFMA k-slices per stage
  constexpr int L = C::kDmaPerStage;
#pragma unroll
  for (int v = -C::kLead; v < 0; ++v)
#pragma unroll
    for (int d = 0; d < L; ++d) issue_group_one(v, d);

  const int frow = lane & 31;  // fragment row (A) / column (B)
  // A combine that reads X (one orientation kept, row-major output every iteration but
  // the last of a transposed bucket) passes its operands to the MFMA the other way
  // round, so its accumulators hold the transposed layout: a lane keeps one row of the
  // tile and runs of 4 columns, so the epilogue stages the row-major tile and its
  // output leaves straight from the staged rows, without transposing LDS reads (the
  // products are the same, summed over k in the same order).  Measured 2-2.4 % less
  // Newton-Schulz time on the 12-, 20- and 24-layer workloads than the plain layout;
  // the combine that keeps X^T writes both orientations every iteration and keeps the
  // plain layout.
  constexpr bool kSwap = (kEpi == kCombine) && C::kCombineReadsX;
  const int fkh = lane >> 5;   // which 8-wide half of a 16-wide k slice

  // wait until stage `st` has landed (called once groups up to st - 1 are issued):
  // the DMAs issued after its last one may stay in flight
  auto wait_stage = [&](int st) {
    if constexpr (C::SB != C::SA) {
      // the shallow operand's stage st went out first in group st - 1; only the deep
      // operand's stage st + 1 follows it
      constexpr int kDeep = C::kBFirst ? C::kDmaA : C::kDmaB;
      if (st + 1 < nk) wait_vmcnt<kDeep>(); else wait_vmcnt<0>();
      return;
    }
    const int pending = min(C::STAGES - 2, nk - 1 - st);
    static_assert(C::STAGES <= 5 && 3 * L < 64, "vmcnt range");
    if constexpr (C::STAGES >= 5) {
      if (pending >= 3) { wait_vmcnt<3 * L>(); return; }
    }
    if constexpr (C::STAGES >= 4) {
      if (pending >= 2) { wait_vmcnt<2 * L>(); return; }
    }
    if constexpr (C::STAGES >= 3) {
      if (pending >= 1) { wait_vmcnt<L>(); return; }
    }
    wait_vmcnt<0>();
  };
  auto load_frags = [&](int kt, int kk, bf16x8 (&af)[C::WTM], bf16x8 (&bfr)[C::WTN]) {
    const unsigned short* as = smem + (kt % C::SA) * C::kAElems;
    const unsigned short* bs = smem + C::kBBase + (kt % C::SB) * C::kBElems;
    const int ch = kk * 2 + fkh;
#pragma unroll
    for (int i = 0; i < C::WTM; ++i) {
      const int r = wm * (C::WTM * 32) + i * 32 + frow;
      af[i] = *reinterpret_cast<const bf16x8*>(as + r * C::BK + swz<C::BK>(r, ch) * 8);
    }
#pragma unroll
    for (int j = 0; j < C::WTN; ++j) {
      if constexpr (kBT) {
        // k rows kk*16 + 8*(lane/32) + 0..7 of column wn*.. + j*32 + lane%32, as two
        // transposing reads of 4 rows each (same k order as the A fragment)
        const int g16 = lane >> 4, sl = lane & 15;
        const int col = wn * (C::WTN * 32) + j * 32 + 16 * (g16 & 1) + 4 * (sl & 3);
        const int row = kk * 16 + 8 * (g16 >> 1) + (sl >> 2);
        const s16x4 lo = lds_read_tr(bs + row * C::BN + swz_kn(row, col >> 3) * 8 + (col & 7));
        const s16x4 hi =
            lds_read_tr(bs + (row + 4) * C::BN + swz_kn(row + 4, col >> 3) * 8 + (col & 7));
        const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        bfr[j] = __builtin_bit_cast(bf16x8, both);
      } else {
        const int r = wn * (C::WTN * 32) + j * 32 + frow;
        bfr[j] = *reinterpret_cast<const bf16x8*>(bs + r * C::BK + swz<C::BK>(r, ch) * 8);
      }
    }
  };

  // Fragments are double-buffered: the LDS reads of k-slice kk+1 are issued before the
  // MFMAs of slice kk, and across a stage boundary the barrier wait and the first
  // reads of the next stage sit before the MFMAs of the last slice, so the matrix
  // cores keep working while the block synchronises.
  // the polynomial's b R term captured from the B stage (see Cfg::kCaptureAux)
  u32x2 cap[C::kCaptureAux ? C::WTM : 1][C::WTN][4];
  auto capture = [&](int kt_stage) {
    if constexpr (C::kCaptureAux && kEpi == kPoly) {
      const unsigned short* bs = smem + C::kBBase + (kt_stage % C::SB) * C::kBElems;
      const int k0 = kt_stage * C::BK;
#pragma unroll
      for (int i = 0; i < C::WTM; ++i) {
        const int rbase = static_cast<int>(m0) + wm * (C::WTM * 32) + i * 32;  // 32 rows of i
        if (rbase >= k0 && rbase < k0 + C::BK) {
#pragma unroll
          for (int j = 0; j < C::WTN; ++j) {
            const int jl = wn * (C::WTN * 32) + j * 32 + (lane & 31);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int kl = rbase - k0 + 8 * q + 4 * fkh;  // local k of rows gi0..gi0+3
              cap[i][j][q] = *reinterpret_cast<const u32x2*>(
                  bs + jl * C::BK + swz<C::BK>(jl, kl >> 3) * 8 + (kl & 4));
            }
          }
        }
      }
    }
  };
  bf16x8 fa[2][C::WTM], fb[2][C::WTN];
  wait_stage(0);
  stage_barrier();
  load_frags(0, 0, fa[0], fb[0]);
  capture(0);
  // The wait for stage kt + 1 once every DMA after it is still in flight (the steady
  // state of wait_stage, with no branch on the stage index).
  auto wait_next_steady = [&]() {
    if constexpr (C::SB != C::SA) {
      constexpr int kDeep = C::kBFirst ? C::kDmaA : C::kDmaB;
      wait_vmcnt<kDeep>();
    } else if constexpr (C::STAGES >= 3) {
      wait_vmcnt<(C::STAGES - 2) * L>();
    } else {
      wait_vmcnt<0>();
    }
  };
  // One stage.  kSteady: every DMA group of the ring still has a stage to load and a
  // next stage exists, so the stage is straight-line code (no branch on kt): the
  // compiler's wait counts are then exact and the next stage's first fragment reads
  // overlap the last k-slice's MFMAs as intended, where a branch around them made it
  // wait for every LDS read before that slice's second MFMA.  kSpread: the DMA issue
  // pattern (chosen once per block).
  auto run_stage = [&](int kt, auto steady_tag, auto spread_tag) {
    constexpr bool kSteady = decltype(steady_tag)::value;
    constexpr bool kSpread = decltype(spread_tag)::value;
    auto issue = [&](int d) {
      if constexpr (kSteady) issue_one(kt + (is_a(d) ? C::LA : C::LB), d);
      else issue_group_one(kt, d);
    };
    const bool load_next = kSteady || kt + (C::LA < C::LB ? C::LA : C::LB) < nk;
    if constexpr (!kSpread) {
      if (load_next) {
#pragma unroll
        for (int d = 0; d < L; ++d) issue(d);
      }
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int cur = kk & 1;
      constexpr int kHalf = KK / 2 > 0 ? KK / 2 : 1;
      constexpr int kPer = (C::kDmaPerStage + kHalf - 1) / kHalf;
      if constexpr (kSpread) {
        if (load_next && kk < kHalf) {
#pragma unroll
          for (int e = 0; e < kPer; ++e)
            if (kk * kPer + e < C::kDmaPerStage) issue(kk * kPer + e);
        }
      }
      if (kk + 1 < KK) {
        load_frags(kt, kk + 1, fa[cur ^ 1], fb[cur ^ 1]);
      } else if (kSteady || kt + 1 < nk) {
        // stage kt+1 has landed and every wave's reads of this stage are done
        if constexpr (kSteady) wait_next_steady();
        else wait_stage(kt + 1);
        stage_barrier();
        load_frags(kt + 1, 0, fa[cur ^ 1], fb[cur ^ 1]);
        capture(kt + 1);
      }
#pragma unroll
      for (int i = 0; i < C::WTM; ++i)
#pragma unroll
        for (int j = 0; j < C::WTN; ++j)
          acc[i][j] = kSwap ? mfma_32x32x16<kTy>(fb[cur][j], fa[cur][i], acc[i][j])
                            : mfma_32x32x16<kTy>(fa[cur][i], fb[cur][j], acc[i][j]);
    }
    if constexpr ((KK & 1) == 1) {
      // odd slice count: the next stage's first fragments landed in buffer 1
#pragma unroll
      for (int i = 0; i < C::WTM; ++i) fa[0][i] = fa[1][i];
#pragma unroll
      for (int j = 0; j < C::WTN; ++j) fb[0][j] = fb[1][j];
    }
  };
  // steady stages while every DMA group and the next stage exist, then the last ones
  constexpr int kTail = C::kLead > C::STAGES ? C::kLead : C::STAGES;
  auto run_all = [&](auto spread_tag) {
    int kt = 0;
    for (; kt < nk - kTail; ++kt) run_stage(kt, std::true_type{}, spread_tag);
    for (; kt < nk; ++kt) run_stage(kt, std::false_type{}, spread_tag);
  };
  if constexpr (C::BM < 192) {
    run_all(std::false_type{});  // 128-tiles never spread their DMAs
  } else {
    if (args.spread) run_all(std::true_type{});
    else run_all(std::false_type{});
  }

  // ---------------- epilogue ----------------
  // MFMA 32x32 accumulator layout: lane holds column (lane & 31) of the 32x32 tile and
  // rows 8*(r/4) + 4*(lane/32) + r%4 for r = 0..15, i.e. four runs of 4 rows (the
  // combine, kSwap: row (lane & 31) and four runs of 4 columns).
  // The polynomial's b R term is read from R's transposed position (R is symmetric),
  // where a lane's 4 consecutive rows are 8 contiguous bytes, and a is added on the
  // diagonal; the Gram and the combine only scale their accumulators.
  const bool mirror = (kEpi != kCombine) && (ti != tj);
  // the combine may skip either orientation (the last iteration keeps only the one
  // the update reads)
  const bool need_t = (kEpi == kCombine) ? (args.C2 != nullptr) : mirror;
  const bool need_c = (kEpi != kCombine) || (args.C != nullptr);

  // 1. final values in fp32, in place in the accumulators
  if constexpr (kEpi == kPoly) {
    const unsigned short* auxT = args.aux + batch * args.strideAux;
    const bool diag_tile = ti == tj;
    constexpr int kHalves = C::WTM >= 2 ? 2 : 1;  // aux loads in two batches (registers)
#pragma unroll
    for (int hh = 0; hh < kHalves; ++hh) {
      constexpr int kI = C::WTM / kHalves;
      u32x2 ax[kI][C::WTN][4];
#pragma unroll
      for (int ii = 0; ii < kI; ++ii)
#pragma unroll
        for (int j = 0; j < C::WTN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if constexpr (C::kCaptureAux) {
              ax[ii][j][q] = cap[hh * kI + ii][j][q];
            } else {
              // R[gi0 + e][gj] = R[gj][gi0 + e]: 8 contiguous bytes
              const int i = hh * kI + ii;
              const int64_t gj = n0 + wn * (C::WTN * 32) + j * 32 + (lane & 31);
              const int64_t gi0 = m0 + wm * (C::WTM * 32) + i * 32 + 8 * q + 4 * fkh;
              ax[ii][j][q] = *reinterpret_cast<const u32x2*>(auxT + gj * args.ldaux + gi0);
            }
          }
#pragma unroll
      for (int ii = 0; ii < kI; ++ii) {
        const int i = hh * kI + ii;
#pragma unroll
        for (int j = 0; j < C::WTN; ++j) {
          const int jl = wn * (C::WTN * 32) + j * 32 + (lane & 31);
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int il = wm * (C::WTM * 32) + i * 32 + 8 * q + 4 * fkh + e;
              const unsigned int w = ax[ii][j][q][e >> 1];
              const float t = from16<kTy>(static_cast<unsigned short>((e & 1) ? (w >> 16) : (w & 0xffffu)));
              // one rounding order for every tile shape: left to the compiler, the
              // sum of two products was fused either way round depending on the
              // instantiation, and tile shapes differed in the last bit
              float v = __builtin_fmaf(args.beta, acc[i][j][q * 4 + e], args.alpha * t);
              if (diag_tile && il == jl) v += args.diag;
              acc[i][j][q * 4 + e] = v;
            }
        }
      }
    }
  } else if (args.scale || args.post != 0.0f) {
    // first iteration: R = (inv U)(inv U)^T = inv^2 U U^T, X1 = P (inv U) = inv P U;
    // and the Gram-space route's constant factors of its fp16 scaling
    const float sc = args.scale ? args.scale[batch] : 1.0f;
    const float f = ((kEpi == kGram) ? sc * sc : sc) * (args.post != 0.0f ? args.post : 1.0f);
#pragma unroll
    for (int i = 0; i < C::WTM; ++i)
#pragma unroll
      for (int j = 0; j < C::WTN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] *= f;
  }

  // 2. the tile goes through LDS (16-bit) once, staged in the orientation the
  // accumulator layout writes 8 bytes at a time: the transposed tile [BN][BM] for the
  // plain layout (a lane's 4 consecutive rows), the row-major tile [BM][BN] for the
  // swapped one (its 4 consecutive columns).  Rows of the staged tile leave with
  // 16-byte stores as the orientation they hold; the other orientation is read out of
  // the same staging with the transposing LDS loads (ds_read_b64_tr_b16), 16 bytes of
  // one of its rows per lane from two of them.  Staging both orientations in turn
  // instead took a second pass of 2-byte LDS writes and two more barriers.  The output
  // stores are non-temporal (streaming): 1.5-3 % less Newton-Schulz time on the 12- and
  // 20-layer workloads, no change on the larger ones.
  if (!need_c && !need_t) return;
  __syncthreads();  // every wave is done reading the operand stages
  // staged tile: kSR rows of kSW elements; chunk c of row r at sphys(c, r)
  constexpr int kSR = kSwap ? C::BM : C::BN;
  constexpr int kSW = kSwap ? C::BN : C::BM;
  constexpr int kSChunks = kSW / 8;
  auto sphys = [](int c, int r) {
    if constexpr (kSwap) return c ^ (r % kSChunks);
    else return tswz<kSChunks>(c, r);
  };
  unsigned short* St = smem;
#pragma unroll
  for (int i = 0; i < C::WTM; ++i)
#pragma unroll
    for (int j = 0; j < C::WTN; ++j) {
      // kSwap: row rl of the product, columns c0 .. c0 + 3; plain: column jl of the
      // product (a row of the staged transpose), rows c0 .. c0 + 3
      const int r = kSwap ? wm * (C::WTM * 32) + i * 32 + (lane & 31)
                          : wn * (C::WTN * 32) + j * 32 + (lane & 31);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c0 = kSwap ? wn * (C::WTN * 32) + j * 32 + 8 * q + 4 * fkh
                             : wm * (C::WTM * 32) + i * 32 + 8 * q + 4 * fkh;
        u32x2 packed;
        packed[0] = static_cast<unsigned>(to16<kTy>(acc[i][j][q * 4 + 0])) |
                    (static_cast<unsigned>(to16<kTy>(acc[i][j][q * 4 + 1])) << 16);
        packed[1] = static_cast<unsigned>(to16<kTy>(acc[i][j][q * 4 + 2])) |
                    (static_cast<unsigned>(to16<kTy>(acc[i][j][q * 4 + 3])) << 16);
        *reinterpret_cast<u32x2*>(St + r * kSW + sphys(c0 >> 3, r) * 8 + (c0 & 4)) = packed;
      }
    }
  __syncthreads();
  if constexpr (kEpi == kGram && C::BM == C::BN && !kSwap) {
    if (args.symmetrize && ti == tj) {
      // A B^T with A != B (a product of two commuting symmetric matrices) is symmetric
      // only up to rounding; the off-diagonal tiles are mirrored whole, and a diagonal
      // tile takes its upper triangle from its lower one, so the stored matrix is
      // exactly symmetric.  Staged transposed: C[o][x] is St[x][o], so for x > o
      // St[x][o] takes St[o][x] (reads above the staged diagonal, writes below it).
      for (int idx = tid; idx < C::BM * C::BN; idx += C::kThreads) {
        const int x = idx / kSW, o = idx - x * kSW;
        if (x > o)
          St[x * kSW + sphys(o >> 3, x) * 8 + (o & 7)] = St[o * kSW + sphys(x >> 3, o) * 8 + (x & 7)];
      }
      __syncthreads();
    }
  }
  // the orientation the staging holds: its rows, 16 bytes per lane
  const bool direct = kSwap ? need_c : need_t;
  if (direct) {
    unsigned short* D = kSwap ? args.C + batch * args.strideC : args.C2 + batch * args.strideC2;
    const int64_t ld = kSwap ? args.ldc : args.ldc2;
    const int64_t r0 = kSwap ? m0 : n0, col0 = kSwap ? n0 : m0;
    constexpr int kAll = kSR * kSChunks;
    static_assert(kAll % C::kThreads == 0, "epilogue copy");
#pragma unroll
    for (int it = 0; it < kAll / C::kThreads; ++it) {
      const int idx = tid + it * C::kThreads;
      const int row = idx / kSChunks;
      const int c = idx - row * kSChunks;
      const u32x4 v = *reinterpret_cast<const u32x4*>(St + row * kSW + sphys(c, row) * 8);
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(D + (r0 + row) * ld + col0 + c * 8));
    }
  }
  // the other orientation: out[o][x] = St[x][o], o < kSW, x < kSR.  A 16-lane group
  // takes 4 rows o = 4 oq + b of it and 4 chunks x0 = 8 (4 xq + a) (lane 4 a + b) per
  // pair of transposing reads: source lane 4 e + a addresses St[x0 + e][4 oq .. + 3]
  // (then St[x0 + 4 + e]), and lane 4 a + b receives element b of those 4 lanes' runs,
  // i.e. out[4 oq + b][x0 + e] (then x0 + 4 + e).
  const bool other = kSwap ? need_t : need_c;
  if (other) {
    unsigned short* D = kSwap ? args.C2 + batch * args.strideC2 : args.C + batch * args.strideC;
    const int64_t ld = kSwap ? args.ldc2 : args.ldc;
    const int64_t r0 = kSwap ? n0 : m0, col0 = kSwap ? m0 : n0;
    constexpr int kXQ = kSR / 32;          // chunk quads per output row
    constexpr int kTasks = (kSW / 4) * kXQ;  // (row quad, chunk quad) per 16-lane group
    constexpr int kGroups = C::kThreads / 16;
    static_assert(kSR % 32 == 0 && kSW % 4 == 0 && kTasks % kGroups == 0, "transposed copy");
    // as a source this lane is 4 e + a (e = gl >> 2, a = gl & 3); as a receiver it is
    // 4 a + b (a = gl >> 2, b = gl & 3)
    const int gl = lane & 15, ga = gl >> 2, gb = gl & 3;
#pragma unroll
    for (int it = 0; it < kTasks / kGroups; ++it) {
      const int task = (tid >> 4) + it * kGroups;
      const int oq = task / kXQ, xq = task - oq * kXQ;
      const int ocol = 4 * oq;                   // the source runs: St[..][ocol .. + 3]
      const int xs = 8 * (4 * xq + gb) + ga;     // this lane's source row, first read
      const s16x4 lo = lds_read_tr(St + xs * kSW + sphys(ocol >> 3, xs) * 8 + (ocol & 4));
      const s16x4 hi =
          lds_read_tr(St + (xs + 4) * kSW + sphys(ocol >> 3, xs + 4) * 8 + (ocol & 4));
      const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      // this lane's output: row 4 oq + gb, chunk 4 xq + ga
      __builtin_nontemporal_store(
          both, reinterpret_cast<s16x8*>(D + (r0 + ocol + gb) * ld + col0 + 8 * (4 * xq + ga)));
    }
  }
}

// Tile shapes.  Big: 256 x 256 per block (160 KiB LDS, one block per CU); the default
// runs 8 waves of 128 x 64 over stages of k = 64 (one barrier per 64 of k), with a ring
// of 3 A stages and 2 B stages: A is loaded two stages ahead, B one.  The 32 KiB the
// third A slot takes is the LDS a 2 + 2 ring leaves unused; with one stage of each
// operand in flight the loads did not cover the fetch latency, and the deeper A ring
// measured 4-5 % faster on 8192-wide Gram sides, 3-5 % at 2048 and 7 % at 1280 (a deeper
// B ring instead: 1-3 % less; 4 waves of 128 x 128, which cut the LDS reads per MFMA by
// a third: 6-9 % slower, one wave per SIMD hides less latency).  Small:
// 128 x 128, 8 waves of 32 x 64, 2 stages of k = 64 (64 KiB, two blocks per CU: four
// waves per SIMD, at most 126 registers each) for Gram sides too short to fill the chip
// (measured 4.5 % faster there than 4 waves of 64 x 64; 8 waves of 64 x 32 or 16 of
// 32 x 32 lose the second block per CU to register use and run 25 % slower; a third A or
// B slot, 80 KiB per block, is no faster there).  The combine reads X with transposing LDS
// loads when the Gram side is at most 2048 (BucketPlan::keeps_xt false), so those
// buckets keep one orientation of X and skip writing and casting X^T; longer Gram sides
// read the stored X^T with b128 loads (two transposing loads per fragment measured
// 15 % slower at m = 8192, where the long contraction makes the X^T write negligible,
// and 2-3 % faster at m = 1280 and 2048).  MA_NS_BIG=1 selects 8 waves over 4 stages of
// k = 32 instead (deeper prefetch, twice the barriers; measured 3-6 % slower).
using Big8K64 = Cfg<256, 256, 64, 2, 4, 3, false, 2>;
using Big8K64X = Cfg<256, 256, 64, 2, 4, 3, true, 2>;  // combine of Gram sides <= 2048
using Big8 = Cfg<256, 256, 32, 2, 4, 4, false>;
using SmallCfg = Cfg<128, 128, 64, 4, 2, 2, true>;
// Combine only: 192 x 256 tiles (8 waves of 96 x 64) for Gram sides padded to a multiple
// of 768, where three-quarter tiles split the work into rounds of the chip with less
// left over (the 12-layer GPT: 1296 256-tiles are 5.06 rounds, 1728 192-row tiles 6.75).
using Mid8X = Cfg<192, 256, 64, 2, 4, 3, true, 2>;

template <class C, int kTy = kTyBf16>
hipError_t launch_cfg(int epi, const GemmTable& t, hipStream_t s) {
  const int blocks = t.start[t.ngroups];
  if (blocks <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(blocks));
  if constexpr (kTy == kTyF16ToBf16) {
    // the Gram-space route's last product only
    if (epi != kCombine) return hipErrorInvalidValue;
    hipLaunchKernelGGL((ns_gemm_kernel<C, kCombine, kTy>), grid, dim3(C::kThreads), 0, s, t);
  } else if constexpr (kTy == kTyF16) {
    // the Gram-space route's symmetric products (gram epilogue) and polynomials
    if (epi == kCombine) return hipErrorInvalidValue;
    if (epi == kPoly)
      hipLaunchKernelGGL((ns_gemm_kernel<C, kPoly, kTy>), grid, dim3(C::kThreads), 0, s, t);
    else
      hipLaunchKernelGGL((ns_gemm_kernel<C, kGram, kTy>), grid, dim3(C::kThreads), 0, s, t);
  } else {
    switch (epi) {
      case kGram: hipLaunchKernelGGL((ns_gemm_kernel<C, kGram>), grid, dim3(C::kThreads), 0, s, t); break;
      case kPoly: hipLaunchKernelGGL((ns_gemm_kernel<C, kPoly>), grid, dim3(C::kThreads), 0, s, t); break;
      default: hipLaunchKernelGGL((ns_gemm_kernel<C, kCombine>), grid, dim3(C::kThreads), 0, s, t); break;
    }
  }
  return hipGetLastError();
}

int big_variant() {
  static const int v = [] {
    const char* e = std::getenv("MA_NS_BIG");
    return e ? std::atoi(e) : 0;
  }();
  return v;
}

int env_int(const char* name, int dflt) {
  const char* e = std::getenv(name);
  return e ? std::atoi(e) : dflt;
}

// Fill the tile-grid and tile-order fields of one group's arguments (bm x bn tiles).
void set_tiles(int epi, GemmArgs& a, const BucketPlan& p, int bm, int bn, const GemmChoice& ch) {
  // Defaults measured on the MI355X (env knobs for tuning, a tuned choice above both):
  // the eight XCDs sharing each matrix when it has at least kSharedMinTiles tiles (each
  // XCD's share then spans two rounds of the blocks it runs at once), else contiguous
  // runs per XCD; bands of 4 row panels for both tile orders, 8 for the combine under
  // the shared order (1.5 % less time on the owner subset's 8192 x 28672 combines, the
  // same on its square one); spread DMA issue for 256-tiles only.
  constexpr int kSharedMinTiles = 512;
  static const int band_combine = env_int("MA_NS_BAND_COMBINE", 0);  // 0: the rule
  static const int band_tri = env_int("MA_NS_BAND_TRI", 4);
  static const int xcd = env_int("MA_NS_XCD", -1);  // XcdOrder, -1: the rule
  static const int spread = env_int("MA_NS_SPREAD", -1);
  if (bm < 192) a.spread = 0;  // measured slower on 128-tiles
  else if (ch.spread >= 0) a.spread = ch.spread ? 1 : 0;
  else a.spread = spread >= 0 ? spread : 1;
  if (epi == kCombine) {
    a.tiles_m = static_cast<int>(p.m_pad / bm);
    a.tiles_n = static_cast<int>(p.n_pad / bn);
    a.tiles_per_batch = a.tiles_m * a.tiles_n;
  } else {
    a.tiles_m = a.tiles_n = static_cast<int>(p.m_pad / bm);
    a.tiles_per_batch = a.tiles_m * (a.tiles_m + 1) / 2;
  }
  // configuration value (1 runs, 2 round-robin, 3 shared) -> XcdOrder
  if (ch.xcd == 1) a.xcd_remap = kXcdRuns;
  else if (ch.xcd == 2) a.xcd_remap = kXcdRoundRobin;
  else if (ch.xcd == 3) a.xcd_remap = kXcdShared;
  else if (xcd >= kXcdRoundRobin && xcd <= kXcdShared) a.xcd_remap = xcd;
  else a.xcd_remap = a.tiles_per_batch >= kSharedMinTiles ? kXcdShared : kXcdRuns;
  if (ch.band > 0) a.band = ch.band;
  else if (epi != kCombine) a.band = band_tri;
  else if (band_combine > 0) a.band = band_combine;
  else a.band = a.xcd_remap == kXcdShared ? 8 : 4;
}

// 256-tile kernel of the Gram-side products and of the X^T-reading combine: the 4-stage
// k = 32 pipeline when chosen (or forced by MA_NS_BIG=1), else the 3 + 2 ring of k = 64
bool use_big8(int pipeline) { return pipeline == 2 || (pipeline == 0 && big_variant() == 1); }

TileShape shape_of(TileCfg cfg, int pipeline) {
  switch (cfg) {
    case kTileBig:
      return use_big8(pipeline) ? TileShape{Big8::BM, Big8::BN, Big8::BK, Big8::kCombineReadsX}
                                : TileShape{Big8K64::BM, Big8K64::BN, Big8K64::BK,
                                            Big8K64::kCombineReadsX};
    case kTileBigX: return TileShape{Big8K64X::BM, Big8K64X::BN, Big8K64X::BK, Big8K64X::kCombineReadsX};
    case kTileMidX: return TileShape{Mid8X::BM, Mid8X::BN, Mid8X::BK, Mid8X::kCombineReadsX};
    default: return TileShape{SmallCfg::BM, SmallCfg::BN, SmallCfg::BK, SmallCfg::kCombineReadsX};
  }
}

hipError_t launch_table(int epi, GemmTable& t, TileCfg cfg, int pipeline, int ty, hipStream_t s) {
  // the fp16 kernels exist for the default pipeline and the 256 and 128 tiles (the
  // configuration search may still name the others: they run as these)
  if (ty != kTyBf16) {
    if (cfg == kTileMidX) cfg = kTileBigX;
    pipeline = 1;
  }
  // longest contraction first, so the blocks with the most work are dispatched first
  for (int i = 1; i < t.ngroups; ++i)
    for (int j = i; j > 0 && t.g[j].kdim > t.g[j - 1].kdim; --j) {
      const GemmArgs tmp = t.g[j];
      t.g[j] = t.g[j - 1];
      t.g[j - 1] = tmp;
    }
  t.start[0] = 0;
  for (int i = 0; i < t.ngroups; ++i)
    t.start[i + 1] =
        t.start[i] + gemm_group_blocks(t.g[i].tiles_per_batch, t.g[i].tiles_k, t.g[i].xcd_remap);
  for (int i = t.ngroups + 1; i <= kMaxGemmGroups; ++i) t.start[i] = t.start[t.ngroups];
  if (LaunchRecorder* r = launch_recorder()) {
    r->gemm(epi, shape_of(cfg, pipeline), t);
    return hipSuccess;
  }
  if (ty == kTyF16) {
    if (cfg == kTileBig) return launch_cfg<Big8K64, kTyF16>(epi, t, s);
    if (cfg == kTileSmall) return launch_cfg<SmallCfg, kTyF16>(epi, t, s);
    return hipErrorInvalidValue;
  }
  if (ty == kTyF16ToBf16) {
    if (cfg == kTileBig) return launch_cfg<Big8K64, kTyF16ToBf16>(epi, t, s);
    if (cfg == kTileBigX) return launch_cfg<Big8K64X, kTyF16ToBf16>(epi, t, s);
    return launch_cfg<SmallCfg, kTyF16ToBf16>(epi, t, s);
  }
  if (cfg == kTileBig)
    return use_big8(pipeline) ? launch_cfg<Big8>(epi, t, s) : launch_cfg<Big8K64>(epi, t, s);
  if (cfg == kTileBigX) return launch_cfg<Big8K64X>(epi, t, s);
  if (cfg == kTileMidX) {
    if (epi != kCombine) return hipErrorInvalidValue;  // not a symmetric tile
    const int blocks = t.start[t.ngroups];
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL((ns_gemm_kernel<Mid8X, kCombine>), dim3(static_cast<unsigned>(blocks)),
                       dim3(Mid8X::kThreads), 0, s, t);
    return hipGetLastError();
  }
  return launch_cfg<SmallCfg>(epi, t, s);
}

// The tile a launch runs: a 128 or 256 choice on a 256-padded phase (a 128-padded one
// only has 128-tiles), else the phase's own; MA_NS_TILE overrides everything.
int chosen_tile(const BucketPlan& p, int choice) {
  if (forced_tile() || p.tile != 256) return p.tile;
  return (choice == 128 || choice == 256) ? choice : p.tile;
}

}  // namespace

bool combine_192_ok(const BucketPlan& p) {
  return p.tile == 256 && !p.keeps_xt && p.m_pad % Mid8X::BM == 0;
}

int64_t tri_tiles_256(int64_t K, int64_t m) {
  const int64_t m256 = (m + 255) / 256;
  return K * m256 * (m256 + 1) / 2;
}

int64_t comb_tiles_256(int64_t K, int64_t m, int64_t n) {
  return K * ((m + 255) / 256) * ((n + 255) / 256);
}

bool fills_256(int64_t tri, int64_t comb) {
  // 256-tiles once the combine tiles fill the chip twice over at one block per CU and
  // the Gram triangle fills it once; smaller problems keep 128-tiles (two blocks per
  // CU, 4x the blocks).  Measured per bucket: 48 x 512 x 2048 runs 19 % faster on
  // 128-tiles (144 Gram tiles at 256), 48 x 768 x 768 14 % faster (432 combine
  // tiles); 80 x 1280 x 1280 12 % faster on 256-tiles, 48 x 2048 x 2048 16 %.
  return comb >= 512 && tri >= 256;
}

int pick_tile(int64_t K, int64_t m, int64_t n) {
  return (m >= kMinGram256 && fills_256(tri_tiles_256(K, m), comb_tiles_256(K, m, n)))
             ? 256 : SmallCfg::BM;
}

hipError_t launch_gram(const NsGroup* g, int n, const float* const* scale,
                       const GemmChoice& ch, hipStream_t s, int ty, float post) {
  const int tile = chosen_tile(*g[0].plan, ch.tile);
  GemmTable t{};
  t.ngroups = n;
  for (int i = 0; i < n; ++i) {
    const BucketPlan& p = *g[i].plan;
    GemmArgs& a = t.g[i];
    a.A = g[i].X; a.B = g[i].X;
    a.lda = a.ldb = p.n_pad;
    a.strideA = a.strideB = p.m_pad * p.n_pad;
    a.kdim = static_cast<int>(p.n_pad);
    a.C = g[i].R; a.C2 = g[i].R;
    a.ldc = a.ldc2 = p.m_pad;
    a.strideC = a.strideC2 = p.m_pad * p.m_pad;
    a.scale = scale ? scale[i] : nullptr;
    a.post = post;
    a.tiles_k = static_cast<int>(p.K);
    set_tiles(kGram, a, p, tile, tile, ch);
  }
  return launch_table(kGram, t, tile == 256 ? kTileBig : kTileSmall, ch.pipeline, ty, s);
}

hipError_t launch_poly(const NsGroup* g, int n, float a_coef, float b, float c,
                       const GemmChoice& ch, hipStream_t s, int ty) {
  const int tile_choice = ch.tile;
  // The polynomial contracts over the Gram side alone.  Where a 256-tile phase's
  // triangles fill less than two rounds of the chip, it runs on 128-tiles (two blocks
  // per CU, four times the blocks) over the same 256-padded layout: measured 17 %
  // faster for the 12-layer GPT's 768-wide buckets (432 tiles at 256).
  int tile = chosen_tile(*g[0].plan, tile_choice);
  if (tile_choice == 0 && tile == 256 && !forced_tile()) {
    int64_t tri = 0;
    for (int i = 0; i < n; ++i) tri += tri_tiles_256(g[i].plan->K, g[i].plan->m_pad);
    if (tri < 512) tile = SmallCfg::BM;
  }
  GemmTable t{};
  t.ngroups = n;
  for (int i = 0; i < n; ++i) {
    const BucketPlan& p = *g[i].plan;
    GemmArgs& a = t.g[i];
    a.A = g[i].R; a.B = g[i].R;
    a.lda = a.ldb = p.m_pad;
    a.strideA = a.strideB = p.m_pad * p.m_pad;
    a.kdim = static_cast<int>(p.m_pad);
    a.C = g[i].P; a.C2 = g[i].P;
    a.ldc = a.ldc2 = p.m_pad;
    a.strideC = a.strideC2 = p.m_pad * p.m_pad;
    a.aux = g[i].R;
    a.ldaux = p.m_pad;
    a.strideAux = p.m_pad * p.m_pad;
    a.alpha = b; a.beta = c; a.diag = a_coef;
    a.tiles_k = static_cast<int>(p.K);
    set_tiles(kPoly, a, p, tile, tile, ch);
  }
  return launch_table(kPoly, t, tile == 256 ? kTileBig : kTileSmall, ch.pipeline, ty, s);
}

hipError_t launch_sym(const SymProd* pr, int n, const GemmChoice& ch, hipStream_t s, int ty) {
  const int tile_choice = ch.tile;
  // contracts over the Gram side like the polynomial: same tile rule
  int tile = chosen_tile(*pr[0].plan, tile_choice);
  if (tile_choice == 0 && tile == 256 && !forced_tile()) {
    int64_t tri = 0;
    for (int i = 0; i < n; ++i) tri += tri_tiles_256(pr[i].plan->K, pr[i].plan->m_pad);
    if (tri < 512) tile = SmallCfg::BM;
  }
  GemmTable t{};
  t.ngroups = n;
  for (int i = 0; i < n; ++i) {
    const BucketPlan& p = *pr[i].plan;
    GemmArgs& a = t.g[i];
    a.A = pr[i].A; a.B = pr[i].B;
    a.lda = a.ldb = p.m_pad;
    a.strideA = a.strideB = p.m_pad * p.m_pad;
    a.kdim = static_cast<int>(p.m_pad);
    a.C = pr[i].C; a.C2 = pr[i].C;
    a.ldc = a.ldc2 = p.m_pad;
    a.strideC = a.strideC2 = p.m_pad * p.m_pad;
    a.symmetrize = 1;
    a.tiles_k = static_cast<int>(p.K);
    set_tiles(kGram, a, p, tile, tile, ch);
  }
  return launch_table(kGram, t, tile == 256 ? kTileBig : kTileSmall, ch.pipeline, ty, s);
}

hipError_t launch_combine(const NsGroup* g, int n, const float* const* scale, bool last,
                          const GemmChoice& ch, hipStream_t s, int ty, float post) {
  // a phase's buckets agree on the tile and on keeping X^T; a 256-tile phase that reads
  // X (no X^T) may also run its combine on 128-tiles (and on 192 x 256 tiles in bf16)
  bool mid = ch.tile == 192 && !forced_tile() && ty == kTyBf16;
  for (int i = 0; i < n && mid; ++i) mid = combine_192_ok(*g[i].plan);
  const int tile = g[0].plan->keeps_xt ? g[0].plan->tile : chosen_tile(*g[0].plan, ch.tile);
  const TileCfg cfg = g[0].plan->keeps_xt ? kTileBig
                      : mid                ? kTileMidX
                      : tile == 256        ? kTileBigX
                                           : kTileSmall;
  GemmTable t{};
  t.ngroups = n;
  for (int i = 0; i < n; ++i) {
    const BucketPlan& p = *g[i].plan;
    GemmArgs& a = t.g[i];
    const bool reads_x = !p.keeps_xt;  // the launched Cfg::kCombineReadsX
    a.A = g[i].P;
    a.lda = p.m_pad;
    a.strideA = p.m_pad * p.m_pad;
    a.strideB = p.m_pad * p.n_pad;
    a.kdim = static_cast<int>(p.m_pad);
    a.ldc = p.n_pad; a.ldc2 = p.m_pad;
    a.strideC = a.strideC2 = p.m_pad * p.n_pad;
    // the last iteration writes only the orientation the update reads (X'^T when the
    // bucket is transposed)
    const bool tr = last && p.transposed;
    if (reads_x) {
      // one orientation: X' row-major, or X'^T (n_pad x m_pad) into the same buffer
      a.B = g[i].X;
      a.ldb = p.n_pad;
      a.C = tr ? nullptr : g[i].Xn;
      a.C2 = tr ? g[i].Xn : nullptr;
    } else {
      a.B = g[i].XT;  // X[i][j] read as X^T[j][i]
      a.ldb = p.m_pad;
      a.C = tr ? nullptr : g[i].Xn;
      a.C2 = (last && !p.transposed) ? nullptr : g[i].XTn;
    }
    a.scale = scale ? scale[i] : nullptr;
    a.post = post;
    a.tiles_k = static_cast<int>(p.K);
    set_tiles(kCombine, a, p, mid ? Mid8X::BM : tile, mid ? Mid8X::BN : tile, ch);
  }
  return launch_table(kCombine, t, cfg, ch.pipeline, ty, s);
}

}  // namespace ma
