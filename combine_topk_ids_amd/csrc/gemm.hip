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
// persistent (one 4-wave workgroup per CU for 256x256 tiles, two for 64x256).
// Items are handed out in rounds: in round r the workgroups of XCD x
// (workgroup ids x, x+8, ... under the round-robin XCD dispatch) take the x-th
// chunk of consecutive items, so each XCD's L2 sees a compact block of GM row
// tiles x (chunk / GM) column blocks.
//
// Per item the k dimension is cut into slices of 32.  Slices travel from
// global memory straight into an NST-slot LDS ring with 16-byte direct-to-LDS
// loads (no staging registers), NST-2 slices ahead, in an XOR-swizzled layout
// that makes the 16-byte fragment reads conflict-free.  While the MFMAs of
// slice k run, the fragments of slice k+1 are read into a second register set
// and slice k+NST's loads are issued, interleaved in 8 chunks so no issue
// queue starves the MFMA pipe.  The MFMAs take the weight fragment as the
// first operand, so each lane's accumulators hold four consecutive output
// columns of one row: the epilogue writes 8 bytes per store.  gate_up puts
// the gate rows [n0, n0+BN/2) and the matching up rows [I+n0, I+n0+BN/2) of
// W1 in one B tile, so each lane holds gate and up accumulators of the same
// (row, column) and applies SiLU(g)*u in registers before the bf16 store.

#include <utility>

#include "common.h"

namespace moe {
namespace {

constexpr int BK = 32;       // k per LDS stage
constexpr int NST = 4;       // LDS stages in the ring (NST-1 stages of loads in flight)
constexpr int kThreads = 256;
constexpr int kXcds = 8;     // MI355X: 8 XCDs, workgroups dispatched round-robin
constexpr int GM = 8;        // row tiles per scheduling group

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
};

typedef __attribute__((address_space(3))) void* lptr_t;

// Direct-to-LDS 16-byte load (gfx950 global_load_lds_dwordx4): lane l's 16 bytes from `src`
// land at LDS byte address m0 + 16*l.  Issued as asm so that the compiler does not add its
// own whole-queue wait before the LDS reads; the kernel waits with counted vmcnt instead.
// Nothing else in these kernels uses m0 (the asm names it as clobbered).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* src, void* lds_wave_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lptr_t)lds_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(src) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ floatx16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const floatx16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS tile: rows of BK bf16 = 4 pieces of 16 bytes; piece c of row r sits at 16-byte slot
// r*4 + (c ^ ((r >> 2) & 3)), so the 16 lanes of a b128 read (16 rows, one piece) hit 16
// distinct 4-bank groups.
__device__ __forceinline__ int slot_of_piece(int r, int c) { return r * 4 + (c ^ ((r >> 2) & 3)); }

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  [&]<int... I>(std::integer_sequence<int, I...>) { (f(std::integral_constant<int, I>{}), ...); }(
      std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// Wait until at most n of this wave's vector memory operations are outstanding, then barrier.
// Written as one asm statement with a memory clobber: the LDS writes of the direct-to-LDS loads
// are invisible to the compiler, so neither the wait nor the reads after it may be reordered.
template <int n>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(n) : "memory");
}

template <int BM, int BN, int WM, int WN, bool kGateUp, int kPerCU>
__global__ __launch_bounds__(kThreads, kPerCU) void k_grouped_gemm(GemmArgs p) {
  static_assert(WM * WN == kThreads / 64, "4 waves");
  constexpr int MS = BM / WM / 32;   // 32-row subtiles per wave
  constexpr int NS = BN / WN / 32;   // 32-column subtiles per wave
  constexpr int AL = BM * 4 / kThreads;  // direct-to-LDS loads per thread per stage (A)
  constexpr int BL = BN * 4 / kThreads;  // (B)
  constexpr int LPS = AL + BL;
  static_assert(!kGateUp || NS % 2 == 0, "gate and up subtiles pair up");
  __shared__ __attribute__((aligned(16))) uint4 As[NST][BM * 4];
  __shared__ __attribute__((aligned(16))) uint4 Bs[NST][BN * 4];

  const int tid = threadIdx.x, wave0 = tid / 64, lane0 = tid % 64;
  // column blocks; the last one may be partial (I or H not a multiple of the block)
  const int32_t ntn = kGateUp ? (p.I + BN / 2 - 1) / (BN / 2) : (p.H + BN - 1) / BN;
  const int32_t ncol = kGateUp ? p.I : p.H;
  const int32_t nrt = *p.num_tiles;
  const int64_t total = (int64_t)((nrt + GM - 1) / GM) * GM * ntn;
  const int per = gridDim.x / kXcds, xcd = blockIdx.x % kXcds, jx = blockIdx.x / kXcds;
  const int nk = p.Kd / BK;

  for (int64_t round = 0;; ++round) {
    const int64_t item = (round * kXcds + xcd) * per + jx;
    if (item >= total) break;
    const int64_t group = item / (GM * ntn), within = item % (GM * ntn);
    const int32_t nt = (int32_t)(within / GM);
    const int32_t mt = (int32_t)(group * GM + within % GM);
    if (mt >= nrt) continue;
    // Per-thread index values are re-derived for every item (through an empty asm) so that
    // the compiler does not hoist their derived addresses out of the item loop, where they
    // would stay live across the whole kernel and spill.
    int lane = lane0, wave = wave0;
    asm volatile("" : "+v"(lane), "+v"(wave));
    const int wm = wave / WN, wn = wave % WN;
    const int2 tile = p.tiles[mt];
    const int32_t el = tile.x, m0 = tile.y;
    const int32_t valid = min(BM, (int32_t)min((int64_t)p.counts[el], p.clamp) - m0);
    const int32_t off = p.offsets[el];
    const int32_t c0 = kGateUp ? nt * (BN / 2) : nt * BN;

    // This thread's direct-to-LDS loads: load i of the wave writes 16-byte slots
    // [(i*4 + wave)*64, +64) of the stage; lane -> (row, piece) through the swizzle.
    // Rows past the tile / columns past the end re-read a valid row: their outputs are
    // never stored, and every load stays inside its tensor.
    const bf16_t* asrc[AL];
    const bf16_t* bsrc[BL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int slot = (i * 4 + wave) * 64 + lane;
      const int r = slot >> 2, c = (slot & 3) ^ ((r >> 2) & 3);
      const int rr = min(r, valid - 1);
      int64_t row;
      if (!kGateUp) row = (int64_t)off + m0 + rr;
      else if (p.perm) row = p.perm[off + m0 + rr] / p.topk;
      else row = el * p.slab + m0 + rr;
      asrc[i] = p.a + row * p.Kd + c * 8;
    }
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      const int slot = (i * 4 + wave) * 64 + lane;
      const int r = slot >> 2, c = (slot & 3) ^ ((r >> 2) & 3);
      int64_t wrow;
      if (kGateUp) {
        const int32_t col = min(c0 + (r < BN / 2 ? r : r - BN / 2), ncol - 1);
        wrow = (int64_t)el * 2 * p.I + (r < BN / 2 ? col : p.I + col);
      } else {
        wrow = (int64_t)el * p.H + min(c0 + r, ncol - 1);
      }
      bsrc[i] = p.w + wrow * p.Kd + c * 8;
    }
    auto issue = [&](int kt) {
      const int s = kt % NST;
#pragma unroll
      for (int i = 0; i < AL; ++i) dma16(asrc[i] + kt * BK, &As[s][(i * 4 + wave) * 64]);
#pragma unroll
      for (int i = 0; i < BL; ++i) dma16(bsrc[i] + kt * BK, &Bs[s][(i * 4 + wave) * 64]);
    };

    floatx16_t acc[MS][NS];
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int j = 0; j < NS; ++j) acc[i][j] = floatx16_t{0};

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

    // Slice pipeline.  Slice k's LDS slot receives its direct-to-LDS loads NST-2 iterations
    // ahead; iteration k waits for slice k+1's loads, barriers, issues slice k+NST-1's loads,
    // reads slice k+1's fragments into the second register set and runs slice k's MFMAs from
    // the first, so LDS reads overlap the MFMAs.  Slice k+NST-1 reuses the slot of slice k-1,
    // whose fragments every wave read (and consumed) before this iteration's barrier.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // previous item's stores, index loads
#pragma unroll
    for (int s = 0; s < NST - 1; ++s)
      if (s < nk) issue(s);
    bf16x8_t fa[BK / 16][MS], fb[BK / 16][NS];  // fragments of the slice being multiplied
    bf16x8_t ga[BK / 16][MS], gb[BK / 16][NS];  // fragments of the next slice, in flight
    auto read_slice = [&](int kt, bf16x8_t (&xa)[BK / 16][MS], bf16x8_t (&xb)[BK / 16][NS]) {
      const uint4* a_s = As[kt % NST];
      const uint4* b_s = Bs[kt % NST];
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int c = ks * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < MS; ++i) xa[ks][i] = *(const bf16x8_t*)&a_s[slot_of_piece(arow0 + i * 32, c)];
#pragma unroll
        for (int j = 0; j < NS; ++j) xb[ks][j] = *(const bf16x8_t*)&b_s[slot_of_piece(brow[j], c)];
      }
    };
    // wait for slice kt (this thread issued slices up to kt + NST - 2 so far)
    auto wait_slice = [&](int kt) {
      const int ahead = min(NST - 2, nk - 1 - kt);  // slices issued after slice kt
      if (ahead >= 3) wait_vm_barrier<3 * LPS>();
      else if (ahead == 2) wait_vm_barrier<2 * LPS>();
      else if (ahead == 1) wait_vm_barrier<LPS>();
      else wait_vm_barrier<0>();
    };
    // The previous slice's fragment reads finished long ago; saying so (lgkmcnt(0), in a form
    // the compiler's wait tracking understands, on every path) keeps it from waiting on the
    // next slice's reads before this slice's MFMAs (lgkmcnt tracks at most 15 operations).
    auto lgkm_drained = [] { __builtin_amdgcn_s_waitcnt(0xC07F); };
    // nk is even (H % 128 == 0, I % 64 == 0): two slices per iteration, alternating fragment
    // sets.  Each slice's work is cut into 8 chunks of (its share of the direct-to-LDS loads of
    // slice kt+NST, two LDS fragment reads of slice kt+1, 1/8 of slice kt's MFMAs) so that no
    // issue queue stalls the MFMA pipe.  The read of slice kt+2 on the last iteration re-reads
    // a slot whose values go unused.
    constexpr int NFR = (BK / 16) * (MS + NS);   // fragment reads per slice
    constexpr int NMF = (BK / 16) * MS * NS;     // MFMAs per slice
    constexpr int NCH = 8;
    static_assert(NFR % NCH == 0 && NMF % NCH == 0, "even chunks");
    // one slice's work with compile-time indices: SET is the fragment set being multiplied,
    // the other set receives slice kt+1
    auto half = [&]<int SET>(int kt, bool load) {
      auto& ca = SET == 0 ? fa : ga;
      auto& cb = SET == 0 ? fb : gb;
      auto& na = SET == 0 ? ga : fa;
      auto& nb = SET == 0 ? gb : fb;
      const uint4* a_n = As[(kt + 1) % NST];
      const uint4* b_n = Bs[(kt + 1) % NST];
      const int sl = (kt + NST) % NST;
      static_for<NCH>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        if (load) {
          static_for<(q + 1) * LPS / NCH - q * LPS / NCH>([&](auto dc) {
            constexpr int d = q * LPS / NCH + decltype(dc)::value;
            if constexpr (d < AL) dma16(asrc[d] + (kt + NST) * BK, &As[sl][(d * 4 + wave) * 64]);
            else dma16(bsrc[d - AL] + (kt + NST) * BK, &Bs[sl][((d - AL) * 4 + wave) * 64]);
          });
        }
        static_for<NFR / NCH>([&](auto fc) {
          constexpr int f = q * NFR / NCH + decltype(fc)::value;
          constexpr int ks = f / (MS + NS), r = f % (MS + NS);
          const int c = ks * 2 + (lane >> 5);
          if constexpr (r < MS) na[ks][r] = *(const bf16x8_t*)&a_n[slot_of_piece(arow0 + r * 32, c)];
          else nb[ks][r - MS] = *(const bf16x8_t*)&b_n[slot_of_piece(brow[r - MS], c)];
        });
        static_for<NMF / NCH>([&](auto mc) {
          constexpr int m = q * NMF / NCH + decltype(mc)::value;
          constexpr int ks = m / (MS * NS), i = (m / NS) % MS, j = m % NS;
          acc[i][j] = mfma32(cb[ks][j], ca[ks][i], acc[i][j]);
        });
      });
    };
    wait_slice(0);
    if (NST - 1 < nk) issue(NST - 1);
    read_slice(0, fa, fb);
    for (int kt = 0; kt < nk; kt += 2) {
      wait_slice(kt + 1);
      lgkm_drained();
      half.template operator()<0>(kt, kt + NST < nk);
      if (kt + 2 < nk) wait_slice(kt + 2);
      lgkm_drained();
      half.template operator()<1>(kt + 1, kt + 1 + NST < nk);
    }
    // every wave is past its last LDS read before the next item's loads overwrite the ring
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

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

template <bool kGateUp>
hipError_t launch(const GemmArgs& a, int32_t bm, hipStream_t stream) {
  const dim3 block(kThreads);
  // 256x256 tiles: one workgroup per CU (128 KB LDS ring); 64x256 tiles: two per CU
  if (bm == 256)
    hipLaunchKernelGGL((k_grouped_gemm<256, 256, 2, 2, kGateUp, 1>), dim3(persistent_grid(1)), block, 0, stream, a);
  else
    hipLaunchKernelGGL((k_grouped_gemm<64, 256, 1, 4, kGateUp, 2>), dim3(persistent_grid(2)), block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int32_t gemm_row_tile(const Geom& g) {
  // expected rows per local expert under even routing: N*K/E
  const int64_t avg = (int64_t)g.N * g.K / g.E;
  return avg >= 512 ? 256 : 64;
}

hipError_t launch_gemm_gate_up(const Geom& g, GemmRows rows, const int32_t* counts, const int32_t* offsets,
                               int64_t count_clamp, const bf16_t* w_gate_up, bf16_t* h, const int2* tiles,
                               const int32_t* num_tiles, int32_t bm, hipStream_t stream) {
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
  return launch<true>(a, bm, stream);
}

hipError_t launch_gemm_down(const Geom& g, const int32_t* counts, const int32_t* offsets, int64_t count_clamp,
                            const bf16_t* h, const bf16_t* w_down, bf16_t* y, int64_t out_slab, const int2* tiles,
                            const int32_t* num_tiles, int32_t bm, hipStream_t stream) {
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
  return launch<false>(a, bm, stream);
}

}  // namespace moe
