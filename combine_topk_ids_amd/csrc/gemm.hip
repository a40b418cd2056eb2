// Grouped expert GEMMs on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16), fp32
// accumulation.
//
// What is computed (FlashInfer "MoE-EP implementation & usage", section 2
// "Call stack": the expert GEMM is a pure per-expert grouped GEMM with no
// routing inside; section 4 "Usage walkthrough": w1 [E, 2I, H], w2 [E, H, I]):
// for local expert e with rows X_e (its received rows, in slot / pick order)
//     h = SiLU(X_e W1_e[0:I]^T) * (X_e W1_e[I:2I]^T)      (gate_up, fused SwiGLU)
//     y = h W2_e^T                                         (down)
// Both operands of both GEMMs are K-contiguous row-major ("NT"), the native
// operand layout of the MFMA: lane l of a 32x32x16 step holds 8 consecutive k
// of one row of each operand, so tiles go from global memory to LDS to
// registers without any transpose or weight shuffle.
//
// Work decomposition.  The device-built tile table lists (expert, first row)
// tiles of BM rows; a work item is (row tile, column block of BN).  The grid is
// persistent: one 4-wave workgroup per CU for 256x256 tiles (each wave
// 128x128, 16x16x32 MFMAs: k_grouped_gemm16), two 4-wave workgroups per CU for
// 64x256 tiles (each wave 64x64, 32x32x16 MFMAs: k_grouped_gemm), and for a gate_up
// GEMM with fewer than two such items per CU two per CU of 64x128 tiles with three k-slice
// stages each (each wave 32x64; twice the items, and two slices in flight).  Items are
// handed out in rounds: in round r the workgroups of XCD x (workgroup ids x,
// x+8, ... under the round-robin XCD dispatch) take the x-th chunk of
// consecutive items, so each XCD's L2 sees a compact block of GM row tiles x
// (chunk / GM) column blocks, and the eight XCDs work on neighbouring blocks of
// the same experts, whose repeated reads the Infinity Cache serves.  GM = 4: an
// XCD's 32 CUs share each activation panel 8 ways and each weight panel 4 ways
// (measured against 8, 2 and 1 row tiles per group: 1% faster than the next).  (Handing
// items out dynamically through per-XCD ticket counters balanced the XCDs'
// finish times but broke this alignment and measured slower.)  The 64-row kernel's groups
// stop at expert boundaries (an expert's last group holds its remaining one to four row tiles),
// so the row tiles that share a weight panel are always neighbouring items (rank-major
// workload, three or four row tiles per expert: L2 hit rate 60% -> 74%, gate_up 87.9 -> 84.0 us,
// down 46.3 -> 43.0 us), and
// a last, partial round is dealt evenly over the eight XCDs (round_item); the narrow gate_up kernel
// instead splits that round's items along K into parts that the workgroups finishing their full
// rounds first take by ticket (rank-major workload: 572 items on 512 workgroups, gate_up 84.2 ->
// 73.6 us; the second workgroup of a CU runs its items about a third slower than the first, so a
// whole tail item on an early finisher used to end after everything else).  The 256x256 kernels
// hand the items of their last three rounds out by ticket (one agent-scope atomic per item, taken
// when the previous item's k-loop ends), so that the XCDs that run faster take more of them: with
// equal static shares the eight XCDs of the prefill workload finished up to 5% apart (prefill
// gate_up 7237 -> 7097 us, down 3871 -> 3745 us).  The 256x256
// kernel issues an item's first loads during the previous item's epilogue, and
// addresses its operands with 32-bit byte offsets from the operand bases (used
// only when every offset fits).  The next item's setup is a dependent chain of
// small loads (tile entry; the expert's count and offset; for gathered A rows,
// the row numbers): each link is issued whole before it is used, and the down
// kernel loads the first two links at the start of the current item so they
// land during its k-loop (the gate_up kernel has no registers to spare for
// that across its SwiGLU epilogue).
//
// Per item the k dimension is cut into slices of 64 (one 128-byte line of
// every A and W row).  Slices travel from global memory straight into LDS
// stages with 16-byte direct-to-LDS loads (no staging registers), in an
// XOR-swizzled layout that makes the 16-byte fragment reads conflict-free.
// The A rows (activations, the operand that misses L2 most) have three stages
// when the tile allows it (3 x 32 KB + 2 x 32 KB = the CU's 160 KB), W two.  A
// slice is multiplied in k steps (two of 32 with 16x16x32 MFMAs, four of 16
// with 32x32x16); the fragments of the next step are read into a second
// register set while the current step's MFMAs run, and the next slice's loads
// are issued right after the barrier that frees their stage (A two slices
// ahead, W one).  Scheduling barriers pin this interleaving so the compiler
// cannot pull a fragment read down next to its first use.  The MFMAs take the
// weight fragment as the first operand, so each lane's accumulators hold four
// consecutive output columns of one row (the 64x256 kernel's epilogue writes
// 8 bytes per store; the 256x256 kernel stages its tile through LDS and stores
// whole 128-byte lines).  gate_up puts the gate rows [n0, n0+BN/2) and the matching up rows
// [I+n0, I+n0+BN/2) of W1 in one B tile, so each lane holds gate and up
// accumulators of the same (row, column) and applies SiLU(g)*u in registers
// before the bf16 store.

#include <algorithm>
#include <utility>

#include "common.h"

namespace moe {
namespace {

constexpr int BK = 64;       // k per LDS stage: one 128-byte line of every row
constexpr int PPR = BK / 8;  // 16-byte pieces per LDS row
constexpr int kXcds = 8;     // MI355X: 8 XCDs, workgroups dispatched round-robin
constexpr int GM = 4;        // row tiles per scheduling group
// Split-K partials of the 256-row kernel: at most this many split items (1.5 x the 256 workgroups of
// the persistent grid), 256 x 256 fp32 each, and four arrival counters (one per wave) per base item
constexpr int kSplitSlots = 384;
// 256-row kernels: the last rounds of items handed out by ticket
constexpr int kDynRounds = 3;
// The narrow 64-row gate_up kernel's split tail: at most this many parts (one fp32 64 x 128 partial
// tile each), arrival counters per wave of each split item, and the parts' ticket counter last
constexpr int kTailParts = 512;
constexpr int kTailPartialFloats = 64 * 128;
constexpr int kTailCounters = kTailParts * 4 + 1;
// Word 3 of a gfx9 raw buffer resource (32-bit data format, no swizzle).
constexpr int kBufferRsrcWord3 = 0x00020000;
typedef unsigned int u4v_t __attribute__((ext_vector_type(4)));

struct GemmArgs {
  // A rows.  gate_up: EM slab rows (a + (e*slab + m) * Kd) or gathered received rows
  // (a + (perm[off + m] / topk) * Kd); down: packed h rows (a + (off + m) * Kd).
  const bf16_t* a;
  const int32_t* perm;
  int32_t topk;
  int64_t slab;
  const int32_t* counts;
  const int32_t* offsets;
  int64_t clamp;
  const bf16_t* w;       // gate_up: [L, 2I, H]; down: [L, H, I]
  bf16_t* out;           // gate_up: h [P, I]; down: y
  int64_t out_slab;      // down: EM slab layout rows per expert (0 = packed)
  const int2* tiles;
  const int32_t* num_tiles;
  int32_t Kd;            // contraction length: H (gate_up) or I (down)
  int32_t I, H;
  // down GEMM with the combine fused in (kCombine): output row m of expert e (packed pick off[e] + m)
  // is added, times its weight, into the token-major output row of its token, with bf16 atomics
  const float* pick_w;   // [P] weight of each pick, in packed (expert-sorted) order
  const int32_t* pick_tok;  // [P] source token of each pick
  bf16_t* out_tok;       // [N, H] token-major output, zeroed before the GEMM
  // split-K of the 256-row kernel (max_split > 1): split ks of an item covers slices
  // [ks * nk / S, (ks + 1) * nk / S); each wave writes its fp32 partial quadrant, and the wave of the
  // split that arrives last (split_cnt) sums the S partials in split order and runs the epilogue
  int32_t max_split;
  float* partial;        // [kSplitSlots, 256 * 256]
  int32_t* split_cnt;    // [kSplitSlots * 4 / 2] arrival counts, zero before the GEMM, reset by the last split
  int32_t* tickets;      // the 256-row kernels: ticket counter of their last rounds (one per GEMM), zero at launch
};

typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
// out[0..1] += (v.lo, v.hi) as two bf16, one packed atomic (global_atomic_pk_add_bf16; the sum is
// rounded to bf16 at each add, in whatever order the adds arrive)
__device__ __forceinline__ void atomic_add_bf16x2(bf16_t* out, uint32_t v) {
  __builtin_amdgcn_global_atomic_fadd_v2bf16((bf16x2v_t*)out, __builtin_bit_cast(bf16x2v_t, v));
}

typedef __attribute__((address_space(3))) void* lptr_t;

// Direct-to-LDS 16-byte load (gfx950 global_load_lds_dwordx4): lane l's 16 bytes from `src`
// land at LDS byte address lds_byte + 16*l (lds_byte is wave-uniform).  Issued as asm so that
// the compiler does not add its own whole-queue wait before the LDS reads; the kernel waits
// with explicit vmcnt instead.  Nothing else in these kernels uses m0 (the asm names it as
// clobbered).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_byte), "v"(src) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ floatx16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const floatx16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS tile: rows of BK bf16 = 8 pieces of 16 bytes; piece c of row r sits at 16-byte slot
// r*8 + (c ^ ((r >> 1) & 7)), so the 16 lanes of a b128 read (16 rows, one piece) hit 16
// distinct 4-bank groups.
// Direct-to-LDS 16-byte load with a scalar base: lane l's 16 bytes from base + voff land at LDS
// byte lds_byte + 16*l (base and lds_byte wave-uniform, voff per lane); m0 is clobbered.
__device__ __forceinline__ void dma16s(const uint8_t* base, uint32_t voff, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_byte), "v"(voff), "s"(base)
               : "memory", "m0");
}

__device__ __forceinline__ int slot_of_piece(int r, int c) { return r * PPR + (c ^ ((r >> 1) & 7)); }

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  [&]<int... I>(std::integer_sequence<int, I...>) { (f(std::integral_constant<int, I>{}), ...); }(
      std::make_integer_sequence<int, N>{});
}

// Item of workgroup (xcd, jx) in round r of a persistent grid of `grid` workgroups (a multiple of
// 8, workgroup b running on XCD b % 8 as the dispatcher deals them): a full round gives each XCD a
// contiguous range of grid/8 items, so that neighbouring items share its L2; the last, partial
// round deals its n items evenly over the eight XCDs (ceil(n/8) each) instead of filling the first
// few (the narrow gate_up GEMM of the rank-major workload: 572 items on 512 workgroups, whose last
// 60 all ran on one XCD; 104 -> 87.5 us).  -1: the workgroup has no item in round r (nor in a later
// one).
__device__ __forceinline__ int64_t round_item(int64_t r, int64_t total, int grid, int xcd, int jx) {
  const int64_t base = r * grid;
  if (base >= total) return -1;
  const int64_t n = total - base < grid ? total - base : grid;
  const int64_t per = (n + kXcds - 1) / kXcds;
  if (jx >= per) return -1;
  const int64_t it = base + xcd * per + jx;
  return it < total ? it : -1;
}

// floor(w / s) for s in 1 .. 4 without a division (s = 3: the multiply-high by ceil(2^33 / 3))
__device__ __forceinline__ int32_t div_upto4(int32_t w, int32_t s) {
  return s == 3 ? (int32_t)(__umulhi((uint32_t)w, 0xAAAAAAABu) >> 1) : w >> (s >> 1);
}
static_assert(GM <= 4, "row-tile groups of at most four tiles");

template <int BM, int BN, int WM, int WN, bool kGateUp, int kPerCU, bool kCombine = false, int NST = 2,
          bool kTail = false>
__global__ __launch_bounds__(WM * WN * 64, kPerCU) void k_grouped_gemm(GemmArgs p) {
  static_assert(!(kGateUp && kCombine), "the combine is fused into the down GEMM");
  constexpr int NW = WM * WN;        // waves
  constexpr int kThreads = NW * 64;
  constexpr int MS = BM / WM / 32;   // 32-row subtiles per wave
  constexpr int NS = BN / WN / 32;   // 32-column subtiles per wave
  constexpr int AL = BM * PPR / kThreads;  // direct-to-LDS loads per thread per stage (A)
  constexpr int BL = BN * PPR / kThreads;  // (B)
  constexpr int LPS = AL + BL;
  static_assert(!kGateUp || NS % 2 == 0, "gate and up subtiles pair up");
  // NST k-slice stages of each operand: slices kt+1 .. kt+NST-1 are in flight while slice kt is read
  static_assert(NST == 2 || NST == 3, "two or three stages");
  __shared__ __attribute__((aligned(16))) uint4 As[NST][BM * PPR];
  __shared__ __attribute__((aligned(16))) uint4 Bs[NST][BN * PPR];

  const int tid = threadIdx.x, wave0 = tid / 64, lane0 = tid % 64;
  // LDS byte offsets (the low 32 bits of a __shared__ object's generic address) of this
  // wave's first 1 KB of each stage; load d of the wave goes d*4 KB further
  const uint32_t swave = (uint32_t)__builtin_amdgcn_readfirstlane(wave0) * 1024u;
  constexpr uint32_t kLoadStride = NW * 1024;  // LDS bytes between a wave's successive loads
  const uint32_t lds_a = (uint32_t)(uintptr_t)&As[0][0] + swave;
  const uint32_t lds_b = (uint32_t)(uintptr_t)&Bs[0][0] + swave;
  constexpr uint32_t kStageA = BM * PPR * 16, kStageB = BN * PPR * 16;
  const int32_t ntn = kGateUp ? (p.I + BN / 2 - 1) / (BN / 2) : (p.H + BN - 1) / BN;
  const int32_t ncol = kGateUp ? p.I : p.H;
  const int32_t nrt = *p.num_tiles;
  const int64_t total = (int64_t)nrt * ntn;
  const int xcd = blockIdx.x % kXcds, jx = blockIdx.x / kXcds;
  const int nk = p.Kd / BK;
  // kTail: the T items of the last, partial round are split along K into S parts each (S a power of
  // two up to 4 with T * S <= grid, at least 8 slices a part), and the parts go to whichever
  // workgroups finish their full rounds first, in ticket order (one agent-scope atomic per part).
  // A part's fp32 partial tile goes to its slot (the part's ticket) with device-scope stores; the
  // wave of an item's last part to arrive sums the S partials in k order (the same sum whichever
  // part that is) and runs the epilogue.  No wave waits for another.
  static_assert(!kTail || (BM * BN == kTailPartialFloats && kGateUp && !kCombine), "split tail: narrow gate_up tiles");
  const int64_t full = total / gridDim.x * gridDim.x;  // items of the full rounds
  const int64_t T = total - full;
  int32_t S = 1;
  if constexpr (kTail)
    while (T > 0 && 2 * S <= 4 && T * 2 * S <= gridDim.x && T * 2 * S <= kTailParts && nk / (2 * S) >= 8) S *= 2;
  const int64_t dealt = S > 1 ? full : total;  // items dealt in rounds
  __shared__ int32_t s_ticket;

  for (int64_t round = 0;; ++round) {
    int64_t item = round_item(round, dealt, gridDim.x, xcd, jx);
    int32_t k0 = 0, nkl = nk, tp = -1;  // the part's first slice, its slices, its ticket
    if (item < 0) {
      if (!kTail || S == 1) break;
      if (threadIdx.x == 0)
        s_ticket = __hip_atomic_fetch_add(&p.split_cnt[kTailCounters - 1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      tp = s_ticket;
      __syncthreads();  // every wave has its ticket before thread 0 takes the next one
      if (tp >= T * S) break;
      item = full + tp / S;
      k0 = (tp % S) * nk / S;
      nkl = (tp % S + 1) * nk / S - k0;
    }
    // Items by expert: expert e's nte row tiles (table entries ts .. ts+nte-1) own items
    // [ts * ntn, (ts + nte) * ntn), in groups of up to GM of its row tiles, each group column block
    // by column block with its row tiles consecutive.  So table entry item / ntn is a tile of the
    // item's expert, and its first row gives ts.
    const int32_t tg = (int32_t)(item / ntn);
    const int2 tile = p.tiles[tg];
    const int32_t el = tile.x;
    const int32_t cnt = p.counts[el], eoff = p.offsets[el];  // issued together
    const int32_t rows_e = (int32_t)min((int64_t)cnt, p.clamp);
    const int32_t nte = (rows_e + BM - 1) / BM;
    const int32_t ts = tg - tile.y / BM;
    const int32_t local = (int32_t)(item - (int64_t)ts * ntn);
    const int32_t grp = tile.y / BM / GM, within = local - grp * (GM * ntn);
    const int32_t sz = min(GM, nte - grp * GM);
    const int32_t nt = div_upto4(within, sz);
    const int32_t m0 = (grp * GM + within - nt * sz) * BM;
    // Per-thread index values are re-derived for every item (through an empty asm) so that
    // the compiler does not hoist their derived addresses out of the item loop, where they
    // would stay live across the whole kernel and spill.
    int lane = lane0, wave = wave0;
    asm volatile("" : "+v"(lane), "+v"(wave));
    const int wm = wave / WN, wn = wave % WN;
    const int32_t valid = min(BM, rows_e - m0);
    const int32_t off = eoff;
    const int32_t c0 = kGateUp ? nt * (BN / 2) : nt * BN;

    // This thread's direct-to-LDS loads: load i of the wave writes 16-byte slots
    // [(i*NW + wave)*64, +64) of the stage; lane -> (row, piece) through the swizzle.
    // Rows past the tile / columns past the end re-read a valid row: their outputs are
    // never stored, and every load stays inside its tensor.  Gathered A rows: all of the
    // thread's row numbers are loaded before any is used.
    const bf16_t* asrc[AL];
    const bf16_t* bsrc[BL];
    int64_t arow[AL];
    if (kGateUp && p.perm) {
#pragma unroll
      for (int i = 0; i < AL; ++i) arow[i] = p.perm[off + m0 + min(((i * NW + wave) * 64 + lane) / PPR, valid - 1)];
#pragma unroll
      for (int i = 0; i < AL; ++i) arow[i] /= p.topk;
    } else {
#pragma unroll
      for (int i = 0; i < AL; ++i) {
        const int rr = min(((i * NW + wave) * 64 + lane) / PPR, valid - 1);
        arow[i] = kGateUp ? el * p.slab + m0 + rr : (int64_t)off + m0 + rr;
      }
    }
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int slot = (i * NW + wave) * 64 + lane;
      const int r = slot / PPR, c = (slot % PPR) ^ ((r >> 1) & 7);
      asrc[i] = p.a + arow[i] * p.Kd + c * 8 + k0 * BK;
    }
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      const int slot = (i * NW + wave) * 64 + lane;
      const int r = slot / PPR, c = (slot % PPR) ^ ((r >> 1) & 7);
      int64_t wrow;
      if (kGateUp) {
        const int32_t col = min(c0 + (r < BN / 2 ? r : r - BN / 2), ncol - 1);
        wrow = (int64_t)el * 2 * p.I + (r < BN / 2 ? col : p.I + col);
      } else {
        wrow = (int64_t)el * p.H + min(c0 + r, ncol - 1);
      }
      bsrc[i] = p.w + wrow * p.Kd + c * 8 + k0 * BK;
    }

    floatx16_t acc[MS][NS];
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int j = 0; j < NS; ++j) acc[i][j] = floatx16_t{0};
    // k order.  When the rows are a multiple of 4 KB apart, an item's slices start at slice
    // nt * nkl / ntn of its range (its column block's share) and wrap around, so that the workgroups in
    // flight read different k offsets of their rows, while the row tiles of one column block, which
    // share its weight panel, keep one order (rank-major workload, rows 8 KB apart: gate_up 72.9 ->
    // 71.8 us; with rows 14 KB apart the rotation measured 0.5% slower).  kel(s): the elements from the
    // range's first to the item's slice s.
    const int32_t krot = (p.Kd * 2) % 4096 == 0 ? (int32_t)((int64_t)nt * nkl / ntn) : 0;
    auto kel = [&](int32_t s) -> int64_t {
      const int32_t k = s + krot;
      return (int64_t)(k >= nkl ? k - nkl : k) * BK;
    };

    // LDS rows of this wave's column subtiles
    int brow[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      if (kGateUp) {
        const int half = j < NS / 2 ? 0 : BN / 2;
        brow[j] = half + wn * (BN / 2 / WN) + (j % (NS / 2)) * 32 + (lane & 31);
      } else {
        brow[j] = wn * (BN / WN) + j * 32 + (lane & 31);
      }
    }
    const int arow0 = wm * (BM / WM) + (lane & 31);

    // Two LDS stages of BK = 64.  A slice is multiplied in four k16 steps; the fragments of
    // step s+1 are read (into the other register set) while step s's MFMAs run.  Slice kt+1's
    // loads are issued during step 3 of slice kt-1, right after the barrier that ends every
    // wave's reads of the stage they overwrite, and waited for at the end of step 2 of slice kt.
    // The previous step's fragment reads are complete before a step's MFMAs (lgkmcnt(0) in a
    // form the compiler's wait tracking understands), and no instruction moves across a
    // chunk boundary (sched_barrier), so every read has a whole step to land.
    bf16x8_t xa[MS], xb[NS], ya[MS], yb[NS];
    auto lgkm_drained = [] { __builtin_amdgcn_s_waitcnt(0xC07F); };
    auto step = [&]<int KS, bool loadB, bool loadA, bool read_next>(int kt, int st) {
      // KS even: multiply set x, read into set y; KS odd: the reverse
      auto& ca = (KS & 1) ? ya : xa;
      auto& cb = (KS & 1) ? yb : xb;
      auto& na = (KS & 1) ? xa : ya;
      auto& nb = (KS & 1) ? xb : yb;
      // the fragments read during this step: (kt, KS+1) from stage st, or (kt+1, 0) from the next
      // stage during step 3
      const int st1 = st + 1 == NST ? 0 : st + 1;
      const int rs = KS == 3 ? st1 : st;
      constexpr int rks = KS == 3 ? 0 : KS + 1;
      const uint4* a_n = As[rs];
      const uint4* b_n = Bs[rs];
      // slice kt's stages are free during step 3: slice kt+NST goes into them
      const int c = rks * 2 + (lane >> 5);
      constexpr int NR = MS + NS;        // fragment reads per step
      constexpr int NM = MS * NS;        // MFMAs per step
      constexpr int NCH = 8;
      static_for<NCH>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (KS == 3 && (loadA || loadB)) {
          static_for<(q + 1) * LPS / NCH - q * LPS / NCH>([&](auto dc) {
            constexpr int d = q * LPS / NCH + decltype(dc)::value;
            if constexpr (d < BL) {
              if constexpr (loadB) dma16(bsrc[d] + kel(kt + NST), lds_b + st * kStageB + d * kLoadStride);
            } else {
              if constexpr (loadA) dma16(asrc[d - BL] + kel(kt + NST), lds_a + st * kStageA + (d - BL) * kLoadStride);
            }
          });
        }
        // the next step's fragment reads go in the first RCH chunks, so the MFMAs of the last
        // NCH - RCH chunks cover their latency before the next step waits for them
        constexpr int RCH = NCH / 2;
        if constexpr ((KS != 3 || read_next) && q < RCH) {
          static_for<(q + 1) * NR / RCH - q * NR / RCH>([&](auto fc) {
            constexpr int f = q * NR / RCH + decltype(fc)::value;
            if constexpr (f < MS) na[f] = *(const bf16x8_t*)&a_n[slot_of_piece(arow0 + f * 32, c)];
            else nb[f - MS] = *(const bf16x8_t*)&b_n[slot_of_piece(brow[f - MS], c)];
          });
        }
        static_for<(q + 1) * NM / NCH - q * NM / NCH>([&](auto mc) {
          constexpr int m = q * NM / NCH + decltype(mc)::value;
          constexpr int i = m / NS, j = m % NS;
          acc[i][j] = mfma32(cb[j], ca[i], acc[i][j]);
        });
      });
      __builtin_amdgcn_sched_barrier(0);
    };

    // prologue: slice 0 (and with three stages slices 1 and 2, A then B of each) issued, slice 0
    // waited for
#pragma unroll
    for (int j = 0; j < (NST == 3 ? 3 : 1); ++j) {
      if (j < nkl) {
#pragma unroll
        for (int i = 0; i < AL; ++i) dma16(asrc[i] + kel(j), lds_a + j * kStageA + i * kLoadStride);
#pragma unroll
        for (int i = 0; i < BL; ++i) dma16(bsrc[i] + kel(j), lds_b + j * kStageB + i * kLoadStride);
      }
    }
    if (NST == 3 && nkl > 2) asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * LPS) : "memory");
    else if (NST == 3 && nkl > 1) asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(LPS) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if constexpr (NST == 2) {
      // two stages: slice 1 goes into stage 1 now (every later slice during step 3 of the slice two
      // before it)
      if (nkl > 1) {
#pragma unroll
        for (int i = 0; i < BL; ++i) dma16(bsrc[i] + kel(1), lds_b + kStageB + i * kLoadStride);
#pragma unroll
        for (int i = 0; i < AL; ++i) dma16(asrc[i] + kel(1), lds_a + kStageA + i * kLoadStride);
      }
    }
    {
      const int c = lane >> 5;
#pragma unroll
      for (int i = 0; i < MS; ++i) xa[i] = *(const bf16x8_t*)&As[0][slot_of_piece(arow0 + i * 32, c)];
#pragma unroll
      for (int j = 0; j < NS; ++j) xb[j] = *(const bf16x8_t*)&Bs[0][slot_of_piece(brow[j], c)];
    }
    // slice kt in stage st.  kLoad: slice kt+NST exists (issued during step 3 into stage st);
    // kWaitN: slice kt+2 exists and is in flight behind slice kt+1 (three stages).
    auto slice = [&]<bool kLoad, bool kRead, bool kWaitN>(int kt, int st) {
      lgkm_drained();
      step.template operator()<0, false, false, true>(kt, st);
      lgkm_drained();
      step.template operator()<1, false, false, true>(kt, st);
      lgkm_drained();
      step.template operator()<2, false, false, true>(kt, st);
      // slice kt+1 has landed (this thread's loads) and every wave has finished reading slice
      // kt's stages (its last fragments were just read into set y)
      if constexpr (kWaitN) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(LPS) : "memory");
      else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      lgkm_drained();
      step.template operator()<3, kLoad, kLoad, kRead>(kt, st);
    };
    int kt = 0, st = 0;
    auto next_st = [&] { st = st + 1 == NST ? 0 : st + 1; };
    // NST == 2: slice kt+2 is issued during slice kt, so no wait leaves a slice in flight
    for (; kt + NST < nkl; ++kt, next_st()) slice.template operator()<true, true, NST == 3>(kt, st);
    if (NST == 3 && kt + 2 < nkl) { slice.template operator()<false, true, true>(kt, st); ++kt; next_st(); }
    if (kt + 1 < nkl) { slice.template operator()<false, true, false>(kt, st); ++kt; next_st(); }
    slice.template operator()<false, false, false>(kt, st);
    // every wave is past its last LDS read (the final step 3 reads nothing) before the next
    // item's loads overwrite the stages
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    if constexpr (kTail) {
      if (tp >= 0) {
        // this wave's quadrant of the part's partial goes to slot tp (16 bytes per lane per store,
        // whole 1 KB lines per wave) with device-scope stores (coherent across the XCDs' L2s for these
        // accesses), complete before the wave counts its arrival
        constexpr int kDeviceScope = 16;  // sc1
        constexpr int Q = MS * NS * 4;    // 16-byte pieces of this lane's accumulators
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            p.partial, 0, (int32_t)(kTailParts * kTailPartialFloats * 4), kBufferRsrcWord3);
        auto piece = [&](int32_t slot, int q) {
          return (int32_t)((slot * kTailPartialFloats + wave * (64 * Q * 4) + q * 256 + lane * 4) * 4);
        };
#pragma unroll
        for (int i = 0; i < MS; ++i)
#pragma unroll
          for (int j = 0; j < NS; ++j)
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
              const floatx4_t v4 = {acc[i][j][4 * c4], acc[i][j][4 * c4 + 1], acc[i][j][4 * c4 + 2], acc[i][j][4 * c4 + 3]};
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4v_t, v4), rs, piece(tp, (i * NS + j) * 4 + c4), 0,
                                                     kDeviceScope);
            }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const int32_t ti = tp / S;
        int32_t arrived = 0;
        if (lane == 0)
          arrived = __hip_atomic_fetch_add(&p.split_cnt[ti * NW + wave], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        arrived = __shfl(arrived, 0, 64);
        if (arrived != S - 1) continue;  // another part of the item is still running
        if (lane == 0) p.split_cnt[ti * NW + wave] = 0;  // ready for the next launch
        floatx16_t sum[MS][NS];
#pragma unroll
        for (int i = 0; i < MS; ++i)
#pragma unroll
          for (int j = 0; j < NS; ++j) sum[i][j] = floatx16_t{0};
        for (int32_t ks = 0; ks < S; ++ks) {
#pragma unroll
          for (int i = 0; i < MS; ++i)
#pragma unroll
            for (int j = 0; j < NS; ++j)
#pragma unroll
              for (int c4 = 0; c4 < 4; ++c4) {
                floatx4_t v4;
                if (ti * S + ks == tp)
                  v4 = floatx4_t{acc[i][j][4 * c4], acc[i][j][4 * c4 + 1], acc[i][j][4 * c4 + 2], acc[i][j][4 * c4 + 3]};
                else
                  v4 = __builtin_bit_cast(floatx4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                         rs, piece(ti * S + ks, (i * NS + j) * 4 + c4), 0, kDeviceScope));
#pragma unroll
                for (int e = 0; e < 4; ++e) sum[i][j][4 * c4 + e] += v4[e];
              }
        }
#pragma unroll
        for (int i = 0; i < MS; ++i)
#pragma unroll
          for (int j = 0; j < NS; ++j) acc[i][j] = sum[i][j];
      }
    }

    // epilogue.  The MFMAs were issued with B as the first operand, so the accumulator holds the
    // transposed tile: lane l has output row l % 32 and, in registers 4g..4g+3, the four
    // consecutive output columns 8g + 4(l/32) + 0..3 -> one 8-byte store per four registers.
    // The values it indexes with pass through an empty asm so that the compiler cannot hoist
    // the address arithmetic above the k-loop (where it would hold registers).
    int lane_e = lane, valid_e = valid, off_e = off, m0_e = m0;
    asm volatile("" : "+v"(lane_e), "+v"(valid_e), "+v"(off_e), "+v"(m0_e));
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      const int row = wm * (BM / WM) + i * 32 + (lane_e & 31);
      if (row >= valid_e) continue;
      if (kGateUp) {
        bf16_t* dst = p.out + (int64_t)(off_e + m0_e + row) * p.I;
#pragma unroll
        for (int j = 0; j < NS / 2; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int32_t col = c0 + wn * (BN / 2 / WN) + j * 32 + 8 * g + 4 * (lane_e >> 5);
            if (col >= p.I) continue;  // I % 64 == 0: four columns are in or out together
            uint2 v;
            v.x = pack_bf16x2(silu_mul(acc[i][j][4 * g + 0], acc[i][j + NS / 2][4 * g + 0]),
                              silu_mul(acc[i][j][4 * g + 1], acc[i][j + NS / 2][4 * g + 1]));
            v.y = pack_bf16x2(silu_mul(acc[i][j][4 * g + 2], acc[i][j + NS / 2][4 * g + 2]),
                              silu_mul(acc[i][j][4 * g + 3], acc[i][j + NS / 2][4 * g + 3]));
            *(uint2*)(dst + col) = v;
          }
        }
      } else if constexpr (kCombine) {
        const int32_t pk = off_e + m0_e + row;
        const float wr = p.pick_w[pk];
        bf16_t* dst = p.out_tok + (int64_t)p.pick_tok[pk] * p.H;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int32_t col = c0 + wn * (BN / WN) + j * 32 + 8 * g + 4 * (lane_e >> 5);
            if (col >= p.H) continue;  // H % 128 == 0
            atomic_add_bf16x2(dst + col, pack_bf16x2(wr * acc[i][j][4 * g + 0], wr * acc[i][j][4 * g + 1]));
            atomic_add_bf16x2(dst + col + 2, pack_bf16x2(wr * acc[i][j][4 * g + 2], wr * acc[i][j][4 * g + 3]));
          }
        }
      } else {
        const int64_t orow = p.out_slab ? (int64_t)el * p.out_slab + m0_e + row : (int64_t)off_e + m0_e + row;
        bf16_t* dst = p.out + orow * p.H;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int32_t col = c0 + wn * (BN / WN) + j * 32 + 8 * g + 4 * (lane_e >> 5);
            if (col >= p.H) continue;  // H % 128 == 0
            uint2 v;
            v.x = pack_bf16x2(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
            v.y = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
            *(uint2*)(dst + col) = v;
          }
        }
      }
    }
  }
}

typedef float floatx4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ floatx4_t mfma16(const bf16x8_t& a, const bf16x8_t& b, const floatx4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 256x256 tile, 4 waves (2x2) of 128x128, 16x16x32 MFMAs.  Operand lane layout: lane l holds 8
// consecutive k (piece l/16 of the step's 4 pieces) of row l%16 of its 16-row operand block; the
// accumulator of W-first MFMAs holds output row l%16 and the 4 consecutive output columns
// 4*(l/16) + 0..3 of the 16x16 block.
template <bool kGateUp, bool kCombine = false, bool kWDeep = false>
__global__ __launch_bounds__(256, 1) void k_grouped_gemm16(GemmArgs p) {
  static_assert(!(kGateUp && kCombine), "the combine is fused into the down GEMM");
  constexpr int BM = 256, BN = 256, NW = 4, kThreads = 256, WN = 2;
  constexpr int MS = 8, NS = 8;  // 16x16 blocks per wave
  constexpr int AL = BM * PPR / kThreads, BL = BN * PPR / kThreads, LPS = AL + BL;
  // Stages: the operand that misses L2 most gets three (loads two slices ahead), the other two.  That
  // is A (gathered activation rows) when the weights are shared by the many row tiles in flight, W
  // when each weight byte is read once by one item (kWDeep: few rows per expert, split-K).  Within a
  // slice the shallow operand's loads go first, so a wait for the deep one's older slice leaves its
  // newest slice in flight.
  constexpr int NSA = kWDeep ? 2 : 3, NSB = kWDeep ? 3 : 2;
  constexpr int SL = kWDeep ? AL : BL, DL = kWDeep ? BL : AL;  // loads per slice: shallow, deep operand
  __shared__ __attribute__((aligned(16))) uint4 As[NSA][BM * PPR];
  __shared__ __attribute__((aligned(16))) uint4 Bs[NSB][BN * PPR];
  const uint32_t swave = (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x / 64) * 1024u;
  // lane and wave numbers made afresh in VGPRs where used (mbcnt, and a copy of the wave's uniform
  // number; volatile, so not hoisted): kept live across the item loop they get spilled, and a
  // reload's wait also waits for the loads in flight
  const int wave0 = (int)(swave >> 10);
  auto lane0f = [] {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
  };
  auto wave0f = [&] {
    int w;
    asm volatile("v_mov_b32 %0, %1" : "=v"(w) : "s"(wave0));
    return w;
  };
  constexpr uint32_t kLoadStride = NW * 1024;
  const uint32_t lds_a = (uint32_t)(uintptr_t)&As[0][0] + swave;
  const uint32_t lds_b = (uint32_t)(uintptr_t)&Bs[0][0] + swave;
  constexpr uint32_t kStageA = BM * PPR * 16, kStageB = BN * PPR * 16;
  const int32_t ntn = kGateUp ? (p.I + BN / 2 - 1) / (BN / 2) : (p.H + BN - 1) / BN;
  const int32_t ncol = kGateUp ? p.I : p.H;
  const int32_t nrt = *p.num_tiles;
  const int32_t base_total = (nrt + GM - 1) / GM * GM * ntn;  // < 2^30: checked on the host
  const int per = gridDim.x / kXcds, xcd = blockIdx.x % kXcds, jx = blockIdx.x / kXcds;
  const int nk = p.Kd / BK;
  // Split-K when there are too few items for the persistent grid: S (a power of two, so that an
  // item's splits are consecutive items) minimising rounds of the grid x (slices per split + 12, the
  // measured cost of the partials' round trip and the last split's sum), with at most kSplitSlots
  // split items and at least 4 slices each.
  // (Only the weight-streaming variant splits: in the other the split bookkeeping would cost registers
  // the 256 accumulators leave no room for, and S is the constant 1.)
  auto choose_split = [&]() -> int32_t {
    int32_t sbest = 1;
    int64_t best = ((int64_t)base_total + gridDim.x - 1) / gridDim.x * nk;
    for (int32_t sp = 2; sp <= p.max_split && (int64_t)base_total * sp <= kSplitSlots && nk / sp >= 4; sp *= 2) {
      const int64_t cost = ((int64_t)base_total * sp + gridDim.x - 1) / gridDim.x * ((nk + sp - 1) / sp + 12);
      if (cost < best) best = cost, sbest = sp;
    }
    return sbest;
  };
  const int32_t S = kWDeep ? choose_split() : 1;
  const int32_t total = base_total * S;
  auto is_padding = [&](int32_t item) {
    const int32_t bitem = item / S;
    const int32_t group = bitem / (GM * ntn), within = bitem % (GM * ntn);
    return group * GM + within % GM >= nrt;
  };
  // Per-item operands: direct-to-LDS load sources, as in k_grouped_gemm (rows / columns past the
  // end re-read a valid one and are never stored), and the output position.
  uint32_t aoff[AL], boff[BL];  // byte offsets from the A and W bases (32-bit: checked on the host)
  const uint8_t* const abase = (const uint8_t*)p.a;
  const uint8_t* const wbase = (const uint8_t*)p.w;
  // An item's wave-uniform metadata: expert, first row, valid rows, the expert's first packed row
  // and the first output column.
  struct Meta {
    int32_t el, m0, valid, off, c0;
    int32_t bitem, ks, kb, nks;  // base item, split, its first slice and its slices
  };
  auto meta = [&](int32_t item) {
    const int32_t bitem = item / S, ks = item % S;
    const int32_t group = bitem / (GM * ntn), within = bitem % (GM * ntn);
    const int32_t nt = (int32_t)(within / GM);
    const int32_t mt = (int32_t)(group * GM + within % GM);
    // scalar loads (through the constant address space: the kernel writes none of these tables), so
    // the values live in SGPRs and the compiler's wait before their first use counts only them
    typedef __attribute__((address_space(4))) const int32_t c_int32;
    const c_int32* const tile = (c_int32*)(uintptr_t)(p.tiles + mt);
    Meta m;
    m.el = tile[0];
    m.m0 = tile[1];
    const int32_t cnt = *(c_int32*)(uintptr_t)(p.counts + m.el), eoff = *(c_int32*)(uintptr_t)(p.offsets + m.el);
    m.valid = min(BM, (int32_t)min((int64_t)cnt, p.clamp) - m.m0);
    m.off = eoff;
    m.c0 = kGateUp ? nt * (BN / 2) : nt * BN;
    m.bitem = bitem;
    m.ks = ks;
    m.kb = ks * nk / S;
    m.nks = (ks + 1) * nk / S - m.kb;
    return m;
  };
  // The item's A row numbers into aoff (rows past the end re-read a valid one and are never
  // stored); for gathered rows these are loads, issued here and consumed by offsets().
  auto rows = [&](const Meta& m) {
    int lane = lane0f(), wave = wave0f();
    asm volatile("" : "+v"(lane), "+v"(wave));
    if (kGateUp && p.perm) {
      // all gathers issued before any is used: one round trip
      int32_t g[AL];
#pragma unroll
      for (int i = 0; i < AL; ++i) g[i] = p.perm[m.off + m.m0 + min(((i * NW + wave) * 64 + lane) / PPR, m.valid - 1)];
#pragma unroll
      for (int i = 0; i < AL; ++i) aoff[i] = (uint32_t)(g[i] / p.topk);
    } else {
#pragma unroll
      for (int i = 0; i < AL; ++i) {
        const int rr = min(((i * NW + wave) * 64 + lane) / PPR, m.valid - 1);
        aoff[i] = kGateUp ? (uint32_t)m.el * (uint32_t)p.slab + (uint32_t)(m.m0 + rr) : (uint32_t)(m.off + m.m0 + rr);
      }
    }
  };
  // Byte offsets of the direct-to-LDS load sources from the A and W bases (32-bit: checked on the
  // host): A from the row numbers rows() left in aoff, W from the expert and the column block.
  auto offsets = [&](const Meta& m) {
    int lane = lane0f(), wave = wave0f();
    asm volatile("" : "+v"(lane), "+v"(wave));
    const uint32_t kd2 = (uint32_t)p.Kd * 2u;
    const uint32_t kofs = (uint32_t)m.kb * (BK * 2);  // the split's first slice
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int slot = (i * NW + wave) * 64 + lane;
      const int r = slot / PPR, c = (slot % PPR) ^ ((r >> 1) & 7);
      aoff[i] = aoff[i] * kd2 + (uint32_t)(c * 16) + kofs;
    }
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      const int slot = (i * NW + wave) * 64 + lane;
      const int r = slot / PPR, c = (slot % PPR) ^ ((r >> 1) & 7);
      uint32_t wrow;
      if (kGateUp) {
        const int32_t col = min(m.c0 + (r < BN / 2 ? r : r - BN / 2), ncol - 1);
        wrow = (uint32_t)m.el * (uint32_t)(2 * p.I) + (uint32_t)(r < BN / 2 ? col : p.I + col);
      } else {
        wrow = (uint32_t)m.el * (uint32_t)p.H + (uint32_t)min(m.c0 + r, ncol - 1);
      }
      boff[i] = wrow * kd2 + (uint32_t)(c * 16) + kofs;
    }
  };
  // the first loads of an item: A(0) and W(0) into stage 0 of each, and slice 1 of the deep operand
  auto issue_first = [&](int32_t nks) {
#pragma unroll
    for (int i = 0; i < AL; ++i) dma16s(abase, aoff[i], lds_a + i * kLoadStride);
#pragma unroll
    for (int i = 0; i < BL; ++i) dma16s(wbase, boff[i], lds_b + i * kLoadStride);
    if (nks > 1) {
      if constexpr (kWDeep) {
#pragma unroll
        for (int i = 0; i < BL; ++i) dma16s(wbase + BK * 2, boff[i], lds_b + kStageB + i * kLoadStride);
      } else {
#pragma unroll
        for (int i = 0; i < AL; ++i) dma16s(abase + BK * 2, aoff[i], lds_a + kStageA + i * kLoadStride);
      }
    }
  };

  // Static rounds: round r < Rs gives this workgroup item (r * kXcds + xcd) * per + jx.  The items of
  // the last kDynRounds rounds go out by ticket to whichever workgroups finish first (not in the
  // split-K variant, whose geometries have few rounds, nor with the combine fused in, where the
  // bookkeeping spilled registers).  Ticket t is item Rs * grid + t counted without the padding items
  // of the last scheduling group, which starts at item lgs and holds glast <= GM real row tiles per
  // column block; the static rounds end before it.
  const int32_t lgs = (nrt - 1) / GM * GM * ntn;
  const int32_t rounds = (total + (int32_t)gridDim.x - 1) / (int32_t)gridDim.x;
  constexpr bool kDyn = !kWDeep && !kCombine;
  int32_t Rs = !kDyn || p.tickets == nullptr ? rounds : max(0, rounds - kDynRounds);
  if (Rs * (int32_t)gridDim.x > lgs) Rs = rounds;  // the static rounds would reach into the last group
  const bool dyn = kDyn && Rs < rounds;
  int32_t round = 0;
  auto next_static = [&]() -> int32_t {
    for (;; ++round) {
      if (kDyn && round >= Rs) return -1;
      const int32_t it = (round * kXcds + xcd) * per + jx;
      if (it >= total) return -1;
      if (!is_padding(it)) return it;
    }
  };
  // the next item's ticket: thread 0 takes it and shares it through a word of A stage 2 (free between the
  // k-loop's last barrier and the epilogue, and before the first item)
  auto next_dynamic = [&]() -> int32_t {
    int32_t* const word = (int32_t*)&As[2][0];
    if (threadIdx.x == 0)
      *word = __hip_atomic_fetch_add(p.tickets, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int32_t t = __builtin_amdgcn_readfirstlane(*word);
    __syncthreads();
    // (lgs and glast recomputed here rather than kept live across the item loop)
    const int32_t lg = (nrt - 1) / GM * GM * ntn, gl = nrt - (nrt - 1) / GM * GM;
    const int32_t d = Rs * (int32_t)gridDim.x + t;
    if (d >= lg + ntn * gl) return -1;
    return d < lg ? d : lg + div_upto4(d - lg, gl) * GM + (d - lg) % gl;
  };
  bool dyn_next = dyn && Rs <= 1;  // the item after the current one comes by ticket
  const int32_t first = dyn && Rs == 0 ? next_dynamic() : next_static();
  if (first < 0) return;
  Meta cur = meta(first);
  rows(cur);
  offsets(cur);
  issue_first(cur.nks);

  for (;;) {
    // down GEMM: the next item's metadata is loaded now and lands during this item's k-loop (the
    // gate_up kernel's SwiGLU epilogue has no registers to spare for it: it loads after the k-loop)
    int32_t nxt = -1;
    Meta nm{};
    if (!kGateUp && !(kDyn && dyn_next)) {
      ++round;
      nxt = next_static();
      if (nxt >= 0) nm = meta(nxt);
    }
    int lane = lane0f(), wave = wave0f();
    asm volatile("" : "+v"(lane), "+v"(wave));
    const int wm = wave / WN, wn = wave % WN;
    const int nk = cur.nks;  // this item's slices (all of K, or its split's)
    floatx4_t acc[MS][NS];
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int j = 0; j < NS; ++j) acc[i][j] = floatx4_t{0, 0, 0, 0};
    int brow[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j)
      brow[j] = kGateUp ? (j < NS / 2 ? 0 : BN / 2) + wn * 64 + (j % (NS / 2)) * 16 + (lane & 15)
                        : wn * 128 + j * 16 + (lane & 15);
    // fused combine: the weights of this lane's epilogue rows (rows past the tile's end read a valid
    // pick and are never stored), loaded now and consumed right after the k-loop, where nothing else
    // is in flight (the compiler's wait for them would otherwise also wait for the next item's first
    // slices, which are issued before the epilogue)
    float w_pick[MS];
    if constexpr (kCombine) {
#pragma unroll
      for (int i = 0; i < MS; ++i)
        w_pick[i] = p.pick_w[cur.off + cur.m0 + min(wm * 128 + i * 16 + (lane & 15), cur.valid - 1)];
    }
    const int arow0 = wm * 128 + (lane & 15);

    bf16x8_t xa[MS], xb[NS], ya[MS], yb[NS];
    auto lgkm_drained = [] { __builtin_amdgcn_s_waitcnt(0xC07F); };
    // step KS (0, 1) multiplies k [32 KS, 32 KS + 32) of slice kt; step 0 reads step 1's fragments,
    // step 1 reads step 0's fragments of slice kt+1 and issues the loads into the freed stages
    auto step = [&]<int KS, bool loadS, bool loadD, bool read_next>(int kt, int sa, int sb) {
      auto& ca = KS ? ya : xa;
      auto& cb = KS ? yb : xb;
      auto& na = KS ? xa : ya;
      auto& nb = KS ? xb : yb;
      const int sa1 = sa + 1 == NSA ? 0 : sa + 1;
      const int sb1 = sb + 1 == NSB ? 0 : sb + 1;
      const uint4* a_n = As[KS ? sa1 : sa];
      const uint4* b_n = Bs[KS ? sb1 : sb];
      const int c = (KS ? 0 : 4) + (lane >> 4);
      constexpr int NR = MS + NS, NM = MS * NS, NCH = 16;
      static_for<NCH>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (KS == 1 && (loadS || loadD)) {
          // into the stages slice kt frees: the shallow operand's slice kt+2, then the deep one's kt+3
          static_for<(q + 1) * LPS / NCH - q * LPS / NCH>([&](auto dc) {
            constexpr int d = q * LPS / NCH + decltype(dc)::value;
            if constexpr (d < SL) {
              if constexpr (loadS) {
                if constexpr (kWDeep) dma16s(abase + (int64_t)(kt + 2) * BK * 2, aoff[d], lds_a + sa * kStageA + d * kLoadStride);
                else dma16s(wbase + (int64_t)(kt + 2) * BK * 2, boff[d], lds_b + sb * kStageB + d * kLoadStride);
              }
            } else {
              if constexpr (loadD) {
                if constexpr (kWDeep) dma16s(wbase + (int64_t)(kt + 3) * BK * 2, boff[d - SL], lds_b + sb * kStageB + (d - SL) * kLoadStride);
                else dma16s(abase + (int64_t)(kt + 3) * BK * 2, aoff[d - SL], lds_a + sa * kStageA + (d - SL) * kLoadStride);
              }
            }
          });
        }
        constexpr int RCH = NCH / 2;
        if constexpr ((KS == 0 || read_next) && q < RCH) {
          static_for<(q + 1) * NR / RCH - q * NR / RCH>([&](auto fc) {
            constexpr int f = q * NR / RCH + decltype(fc)::value;
            if constexpr (f < MS) na[f] = *(const bf16x8_t*)&a_n[slot_of_piece(arow0 + f * 16, c)];
            else nb[f - MS] = *(const bf16x8_t*)&b_n[slot_of_piece(brow[f - MS], c)];
          });
        }
        static_for<(q + 1) * NM / NCH - q * NM / NCH>([&](auto mc) {
          constexpr int m = q * NM / NCH + decltype(mc)::value;
          constexpr int i = m / NS, j = m % NS;
          acc[i][j] = mfma16(cb[j], ca[i], acc[i][j]);
        });
      });
      __builtin_amdgcn_sched_barrier(0);
    };
    // A(0), W(0) and the deep operand's slice 1 were issued before this item's turn (with the
    // previous item's epilogue stores issued after them, these waits may also wait for those stores);
    // now the shallow operand's slice 1 and the deep one's slice 2
    if (nk > 1) {
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(DL) : "memory");
      if constexpr (kWDeep) {
#pragma unroll
        for (int i = 0; i < AL; ++i) dma16s(abase + BK * 2, aoff[i], lds_a + kStageA + i * kLoadStride);
      } else {
#pragma unroll
        for (int i = 0; i < BL; ++i) dma16s(wbase + BK * 2, boff[i], lds_b + kStageB + i * kLoadStride);
      }
    } else {
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    }
    if (nk > 2) {
      if constexpr (kWDeep) {
#pragma unroll
        for (int i = 0; i < BL; ++i) dma16s(wbase + 2 * BK * 2, boff[i], lds_b + 2 * kStageB + i * kLoadStride);
      } else {
#pragma unroll
        for (int i = 0; i < AL; ++i) dma16s(abase + 2 * BK * 2, aoff[i], lds_a + 2 * kStageA + i * kLoadStride);
      }
    }
    {
      const int c = lane >> 4;
#pragma unroll
      for (int i = 0; i < MS; ++i) xa[i] = *(const bf16x8_t*)&As[0][slot_of_piece(arow0 + i * 16, c)];
#pragma unroll
      for (int j = 0; j < NS; ++j) xb[j] = *(const bf16x8_t*)&Bs[0][slot_of_piece(brow[j], c)];
    }
    // slice kt: kLoadS / kLoadD: the shallow operand's slice kt+2 / the deep one's kt+3 exist;
    // kWaitD: the deep operand's slice kt+2 is in flight behind slice kt+1
    auto slice = [&]<bool kLoadS, bool kLoadD, bool kRead, bool kWaitD>(int kt, int sa, int sb) {
      lgkm_drained();
      step.template operator()<0, false, false, true>(kt, sa, sb);
      // the last slice reads nothing more from LDS and loads nothing: no wait, no barrier
      if constexpr (kWaitD) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(DL) : "memory");
      else if constexpr (kRead || kLoadS || kLoadD) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      lgkm_drained();
      step.template operator()<1, kLoadS, kLoadD, kRead>(kt, sa, sb);
    };
    int kt = 0, sa = 0, sb = 0;
    auto next_s = [&] {
      sa = sa + 1 == NSA ? 0 : sa + 1;
      sb = sb + 1 == NSB ? 0 : sb + 1;
    };
    for (; kt + 3 < nk; ++kt, next_s()) slice.template operator()<true, true, true, true>(kt, sa, sb);
    if (kt + 2 < nk) { slice.template operator()<true, false, true, true>(kt, sa, sb); ++kt; next_s(); }
    if (kt + 1 < nk) { slice.template operator()<false, false, true, false>(kt, sa, sb); ++kt; next_s(); }
    slice.template operator()<false, false, false, false>(kt, sa, sb);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if constexpr (kCombine) {
#pragma unroll
      for (int i = 0; i < MS; ++i) asm volatile("" : "+v"(w_pick[i]));
    }
    // Split-K: this wave's fp32 partial quadrant goes out (contiguous per MFMA block), then the
    // wave counts its arrival; the wave whose split arrives last sums the S partials in split order
    // (the same sum whichever split that is) and runs the epilogue; the others skip it.  Device-scope
    // fences order the partial stores before the count and the count before the loads.  Done before
    // the next item's first loads are issued, so that the fences wait for nothing else.
    bool store_out = true;
    if (kWDeep && S > 1) {
      // the partials move with device-scope stores and loads (cache policy sc1: coherent across the
      // XCDs' L2s for these accesses alone), so no L2-wide write-back or invalidate is needed; the
      // stores complete (vmcnt) before the arrival count, which an agent-scope atomic keeps
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          p.partial, 0, (int32_t)(kSplitSlots * BM * BN * 4), kBufferRsrcWord3);
      const int32_t base = ((cur.bitem * S) * (BM * BN) + wave * (64 * MS * NS * 4) + lane * 4) * 4;  // bytes
      constexpr int kDeviceScope = 16;  // sc1
#pragma unroll
      for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4v_t, acc[i][j]), rs,
                                                 base + (cur.ks * (BM * BN) + (i * NS + j) * 256) * 4, 0,
                                                 kDeviceScope);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      int32_t arrived = 0;
      if (lane == 0)
        arrived = __hip_atomic_fetch_add(&p.split_cnt[cur.bitem * NW + wave], 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
      arrived = __shfl(arrived, 0, 64);
      store_out = arrived == S - 1;
      if (store_out) {
        if (lane == 0) p.split_cnt[cur.bitem * NW + wave] = 0;  // ready for the next GEMM
#pragma unroll
        for (int i = 0; i < MS; ++i)
#pragma unroll
          for (int j = 0; j < NS; ++j) {
            floatx4_t t = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int32_t sp = 0; sp < S; ++sp)
              t += sp == cur.ks ? acc[i][j]
                                : __builtin_bit_cast(floatx4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                                    rs, base + (sp * (BM * BN) + (i * NS + j) * 256) * 4,
                                                                    0, kDeviceScope));
            acc[i][j] = t;
          }
      }
    }

    // Next item: its first loads go into stage 0 of each operand and stage 1 of the deep one now, so
    // that they land during this item's epilogue.
    int lane_e = lane, valid_e = cur.valid, off_e = cur.off, m0_e = cur.m0, c0_e = cur.c0, el_e = cur.el;
    asm volatile("" : "+v"(lane_e), "+v"(valid_e), "+v"(off_e), "+v"(m0_e), "+v"(c0_e), "+v"(el_e));
    if (kGateUp || (kDyn && dyn_next)) {
      if (kDyn && dyn_next) {
        nxt = next_dynamic();
      } else {
        ++round;
        nxt = next_static();
      }
      if (nxt >= 0) nm = meta(nxt);
    }
    dyn_next = dyn && (dyn_next || round + 1 >= Rs);
    if (nxt >= 0) {
      rows(nm);
      offsets(nm);
      issue_first(nm.nks);
    }
    if (store_out) {
      // Epilogue through LDS: each wave packs 64 rows of its tile at a time to bf16 into its own 16 KB
      // of the two stages the next item's first loads leave free (A stage 2 and W stage 1, or A 1 and
      // W 2; rows of GP 16-byte granules, granule g of row r at g ^ (r mod GP), so that both the 8-byte
      // writes and the 16-byte reads are conflict-free), then stores whole row segments, 16 bytes per
      // lane: full 128-byte lines instead of 32-byte pieces of 16 rows.
      constexpr int OC = kGateUp ? 64 : 128;  // output columns per wave
      constexpr int GP = OC / 8;              // 16-byte granules per tile row
      constexpr int RPI = 64 / GP;            // tile rows per store instruction
      char* const ot = (char*)(wave < 2 ? &As[kWDeep ? 1 : 2][0] : &Bs[kWDeep ? 2 : 1][0]) + (wave & 1) * 16384;
  #pragma unroll
      for (int half = 0; half < 2; ++half) {
        if (half == 1 && kGateUp) break;
        constexpr int HR = kGateUp ? MS : MS / 2;  // 16-row blocks per pass
  #pragma unroll
        for (int ii = 0; ii < HR; ++ii) {
          const int i = half * HR + ii;
          const int r = ii * 16 + (lane_e & 15);
  #pragma unroll
          for (int j = 0; j < OC / 16; ++j) {
            uint2 v;
            if (kGateUp) {
              v.x = pack_bf16x2(silu_mul(acc[i][j][0], acc[i][j + NS / 2][0]), silu_mul(acc[i][j][1], acc[i][j + NS / 2][1]));
              v.y = pack_bf16x2(silu_mul(acc[i][j][2], acc[i][j + NS / 2][2]), silu_mul(acc[i][j][3], acc[i][j + NS / 2][3]));
            } else if constexpr (kCombine) {
              v.x = pack_bf16x2(w_pick[i] * acc[i][j][0], w_pick[i] * acc[i][j][1]);
              v.y = pack_bf16x2(w_pick[i] * acc[i][j][2], w_pick[i] * acc[i][j][3]);
            } else {
              v.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
              v.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
            }
            const int g = 2 * j + (lane_e >> 5);
            *(uint2*)(ot + r * (GP * 16) + ((g ^ (r & (GP - 1))) * 16) + ((lane_e >> 4) & 1) * 8) = v;
          }
        }
        // the region is this wave's own: its writes only have to land before its reads
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int g = lane_e % GP;
        const int32_t col = c0_e + wn * OC + g * 8;
        // the LDS reads of a batch first, so that they are in flight together (read, wait, store one at
        // a time cost one LDS round trip per 16-byte store), then its stores; the whole pass is one
        // batch except in the split-K variant, whose registers do not hold it
        constexpr int NIT = HR * 16 / RPI;
        constexpr int NB = kWDeep ? 4 : NIT;
        uint4 vv[NIT];
  #pragma unroll
        for (int it = 0; it < NIT; ++it) {
          if (it % NB == 0) {
  #pragma unroll
            for (int b = it; b < it + NB; ++b) {
              const int r = b * RPI + lane_e / GP;
              vv[b] = *(const uint4*)(ot + r * (GP * 16) + ((g ^ (r & (GP - 1))) * 16));
            }
          }
          const int r = it * RPI + lane_e / GP;
          const uint4 v = vv[it];
          const int row = wm * 128 + half * (HR * 16) + r;
          if (row >= valid_e || col >= ncol) continue;
          if (kGateUp) {
            *(uint4*)(p.out + (int64_t)(off_e + m0_e + row) * p.I + col) = v;
          } else if constexpr (kCombine) {
            bf16_t* dst = p.out_tok + (int64_t)p.pick_tok[off_e + m0_e + row] * p.H + col;
            atomic_add_bf16x2(dst + 0, v.x);
            atomic_add_bf16x2(dst + 2, v.y);
            atomic_add_bf16x2(dst + 4, v.z);
            atomic_add_bf16x2(dst + 6, v.w);
          } else {
            const int64_t orow = p.out_slab ? (int64_t)el_e * p.out_slab + m0_e + row : (int64_t)off_e + m0_e + row;
            *(uint4*)(p.out + orow * p.H + col) = v;
          }
        }
        // the next pass rewrites the region only after this pass's reads have returned
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
    }
    if (nxt < 0) break;
    cur = nm;
  }
}

int g_cus[64];

int persistent_grid(int per_cu) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (g_cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cus[dev] = n;
  }
  const int n = g_cus[dev] * per_cu / kXcds * kXcds;
  return n > 0 ? n : kXcds;
}

template <bool kGateUp, bool kCombine = false>
hipError_t launch(const GemmArgs& a, int32_t bm, hipStream_t stream, bool narrow = false) {
  // weight streaming (split-K possible: few rows per expert, each weight byte read by one item):
  // the weights get the three-stage ring
  const bool wdeep = a.max_split > 1;
  // 256x256 tiles: one 4-wave workgroup per CU (160 KB of LDS stages), 16x16x32 MFMAs;
  // 64x256 tiles: two 4-wave workgroups per CU, 32x32x16 MFMAs, two k-slice stages; 64x128 tiles
  // (narrow): two 4-wave workgroups per CU with three stages (72 KB of LDS each; measured against
  // three per CU with two stages on the rank-major workload: gate_up 93.5 -> 87.5 us)
  if (bm == 256 && wdeep)
    hipLaunchKernelGGL((k_grouped_gemm16<kGateUp, kCombine, true>), dim3(persistent_grid(1)), dim3(256), 0, stream, a);
  else if (bm == 256)
    hipLaunchKernelGGL((k_grouped_gemm16<kGateUp, kCombine, false>), dim3(persistent_grid(1)), dim3(256), 0, stream, a);
  else if (narrow && kGateUp && !kCombine && a.partial)
    hipLaunchKernelGGL((k_grouped_gemm<64, 128, 2, 2, kGateUp, 2, kCombine, 3, kGateUp && !kCombine>),
                       dim3(persistent_grid(2)), dim3(256), 0, stream, a);
  else if (narrow)
    hipLaunchKernelGGL((k_grouped_gemm<64, 128, 2, 2, kGateUp, 2, kCombine, 3>), dim3(persistent_grid(2)), dim3(256), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((k_grouped_gemm<64, 256, 1, 4, kGateUp, 2, kCombine>), dim3(persistent_grid(2)), dim3(256), 0, stream,
                       a);
  return hipGetLastError();
}

}  // namespace

bool gemm_offsets_fit_32(const Geom& g) {
  const int64_t lim = (int64_t)1 << 32;
  const int64_t a_rows = g.layout == 0 ? (int64_t)g.L * g.cap : (int64_t)g.rows;  // gate_up A rows
  // work items of the 256x256 kernel (int32 there, with a grid's worth of headroom for the item
  // index one round past the end): at most N*K local picks in 256-row tiles, one partial tile per
  // expert, the group padding, times the column blocks
  const int64_t items = ((int64_t)g.N * g.K / 256 + g.L + GM) * std::max((g.I + 127) / 128, (g.H + 255) / 256);
  return a_rows * g.H * 2 < lim && (int64_t)g.L * 2 * g.I * g.H * 2 < lim &&
         (int64_t)g.N * g.K * g.I * 2 < lim && (int64_t)g.L * g.H * g.I * 2 < lim && items < lim / 4;
}

int32_t gemm_row_tile(const Geom& g) {
  // expected rows per local expert under even routing: N*K/E.  Below 512, 64-row tiles: with a few
  // hundred rows per expert, one 256-row tile per expert (each weight byte read once, split-K for
  // enough items) measured no faster on the rank-major workload (gate_up 94.6 vs 93.3 us) and the
  // split down GEMM slower (69 vs 46 us).
  const int64_t avg = (int64_t)g.N * g.K / g.E;
  return avg >= 512 && gemm_offsets_fit_32(g) ? 256 : 64;
}

// The narrow gate_up tiles (64 x 128): 64-row tiles with fewer than two 64x256 items per CU under even
// routing (a few hundred rows per expert over few experts)
bool gemm_narrow(const Geom& g) {
  const int64_t avg = (int64_t)g.N * g.K / g.E;
  const int64_t items = (int64_t)g.L * ((avg + 63) / 64) * ((g.I + 127) / 128);
  return gemm_row_tile(g) == 64 && g.I > 0 && items < 2 * (int64_t)persistent_grid(1);
}

bool gemm_split_possible(const Geom& g) {
  if (g.I == 0) return false;
  if (gemm_narrow(g)) return true;  // the split tail's partials
  if (gemm_row_tile(g) != 256) return false;
  // expected items of the wider of the two GEMMs under even routing
  const int64_t avg = (int64_t)g.N * g.K / g.E;
  const int64_t tiles = (int64_t)g.L * ((avg + 255) / 256);
  const int64_t items = tiles * std::max((g.I + 127) / 128, (g.H + 255) / 256);
  return items < kSplitSlots;
}

size_t gemm_split_partial_bytes(const Geom& g) {
  return gemm_narrow(g) ? (size_t)kTailParts * kTailPartialFloats * 4 : (size_t)kSplitSlots * 256 * 256 * 4;
}
int32_t gemm_split_counters(const Geom& g) { return gemm_narrow(g) ? kTailCounters : kSplitSlots * 2; }
int32_t gemm_zero_words(const Geom& g) { return kGemmTickets + (gemm_split_possible(g) ? gemm_split_counters(g) : 0); }

hipError_t launch_gemm_gate_up(const Geom& g, GemmRows rows, const int32_t* counts, const int32_t* offsets,
                               int64_t count_clamp, const bf16_t* w_gate_up, bf16_t* h, const int2* tiles,
                               const int32_t* num_tiles, int32_t bm, hipStream_t stream, const SplitBufs& split) {
  GemmArgs a;
  a.a = rows.a;
  a.perm = rows.perm;
  a.topk = rows.K;
  a.slab = rows.slab;
  a.counts = counts;
  a.offsets = offsets;
  a.clamp = count_clamp;
  a.w = w_gate_up;
  a.out = h;
  a.out_slab = 0;
  a.tiles = tiles;
  a.num_tiles = num_tiles;
  a.Kd = g.H;
  a.I = g.I;
  a.H = g.H;
  a.pick_w = nullptr;
  a.pick_tok = nullptr;
  a.out_tok = nullptr;
  a.max_split = split.partial && bm == 256 && !gemm_narrow(g) ? 8 : 1;
  a.partial = bm == 256 || gemm_narrow(g) ? split.partial : nullptr;
  a.split_cnt = split.cnt;
  a.tickets = split.tickets;
  // 64-row tiles with fewer than two 64x256 items per CU under even routing: 64x128 tiles, twice the
  // items, two workgroups per CU, the last partial round split along K when the workspace holds the
  // partials.  (The down GEMM measured slower with these tiles, and so did gate_up with more items.)
  return launch<true>(a, bm, stream, bm == 64 && gemm_narrow(g));
}

hipError_t launch_gemm_down(const Geom& g, const int32_t* counts, const int32_t* offsets, int64_t count_clamp,
                            const bf16_t* h, const bf16_t* w_down, bf16_t* y, int64_t out_slab, const int2* tiles,
                            const int32_t* num_tiles, int32_t bm, hipStream_t stream, const DownCombine& comb,
                            const SplitBufs& split) {
  GemmArgs a;
  a.a = h;
  a.perm = nullptr;
  a.topk = g.K;
  a.slab = 0;
  a.counts = counts;
  a.offsets = offsets;
  a.clamp = count_clamp;
  a.w = w_down;
  a.out = y;
  a.out_slab = out_slab;
  a.tiles = tiles;
  a.num_tiles = num_tiles;
  a.Kd = g.I;
  a.I = g.I;
  a.H = g.H;
  a.pick_w = comb.pick_w;
  a.pick_tok = comb.pick_tok;
  a.out_tok = comb.out;
  a.max_split = split.partial && bm == 256 && !gemm_narrow(g) ? 8 : 1;
  a.partial = split.partial;
  a.split_cnt = split.cnt;
  a.tickets = split.tickets ? split.tickets + 1 : nullptr;  // the gate_up GEMM has the first counter
  return comb.out ? launch<false, true>(a, bm, stream) : launch<false>(a, bm, stream);
}

}  // namespace moe
