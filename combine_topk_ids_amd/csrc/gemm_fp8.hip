// FP8 gate_up expert GEMM on the gfx950 block-scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4,
// E4M3 operands, E8M0 scales), fp32 accumulation, fused SwiGLU, bf16 h.
//
// What is computed: the gate_up product of the expert GEMM (FlashInfer "MoE-EP implementation &
// usage", section 2 "Call stack" and section 4, w1 [E, 2I, H]) on FP8 operands: the received
// rows in the FP8 dispatch format (Mooncake PG/EP guide, "Buffer.dispatch", use_fp8: data plus
// scales) and W1 quantised the same way, one power-of-two scale per row and 128 k.  Value of an
// operand element = e4m3(code) * 2^(scale byte - 127), so
//     h[m][n] = SiLU(sum_k X[m][k] W1[n][k]) * (sum_k X[m][k] W1[I+n][k]).
//
// Layout facts of the scaled MFMA used here (measured on the chip): for the 16x16x128 shape, lane
// l holds row l%16 of its operand; its 32 bytes are k [16g, 16g+16) and k [64+16g, 64+16g+16),
// g = l/16; the scale of (row r, 32-wide k block b) is taken from lane r + 16b.  A slice of 128 k
// is therefore pieces g and g+4 of a 128-byte LDS row, and since one scale covers the whole
// slice, every lane passes the scale of its own row.  The accumulator of a W-first product holds
// output row l%16 and output columns 4*(l/16) + 0..3, as in the bf16 kernel.
//
// Work decomposition and loads as in the bf16 256x256 kernel (persistent, XCD-aware items, the
// last three rounds' items by ticket; direct-to-LDS 16-byte loads of 128-byte row slices into 3 A
// and 2 W stages, XOR-swizzled LDS rows).  Per slice each wave (128x128 outputs, 8x8 MFMA blocks) keeps the slice's eight W
// fragments in registers (read during the previous slice) and streams its eight X fragments, one
// per row of 8 MFMAs; the next slice's W fragments and first X fragment are read meanwhile.
// The scales of four consecutive slices of a row are one aligned 32-bit word, loaded a group of
// four slices ahead with ordinary loads (the compiler's own wait before their first use also waits
// for the tile loads issued after them, a memory latency every four slices; loads issued by asm
// into registers would leave the compiler free to copy or spill those registers before they land).
#include <utility>

#include "common.h"

namespace moe {
namespace {

constexpr int BKB = 128;           // k per slice (bytes of an FP8 row)
constexpr int PPR = BKB / 16;      // 16-byte pieces per LDS row
constexpr int kXcds = 8;
constexpr int GM = 4;
constexpr int kDynRounds = 3;  // rounds of items handed out by ticket at the end

typedef int int8v_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lptr_t;

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// lane l's 16 bytes from src land at LDS byte lds_byte + 16*l (lds_byte wave-uniform); m0 is
// clobbered and used by nothing else here
// lane l's 16 bytes from base + voff land at LDS byte lds_byte + 16*l (base and lds_byte
// wave-uniform, voff per lane); m0 is clobbered and used by nothing else here
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t voff, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_byte), "v"(voff), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ int slot_of_piece(int r, int c) { return r * PPR + (c ^ ((r >> 1) & 7)); }

template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  [&]<int... I>(std::integer_sequence<int, I...>) { (f(std::integral_constant<int, I>{}), ...); }(
      std::make_integer_sequence<int, N>{});
}

struct Fp8Args {
  const uint8_t* a;        // received rows, codes [rows, H]
  const uint8_t* a_scales; // [rows, ss]
  const int32_t* perm;     // RM / FLAT: pick order (row = perm / topk); NULL for EXPERT_MAJOR slabs
  int32_t topk;
  int64_t slab;
  const int32_t* counts;
  const int32_t* offsets;
  int64_t clamp;
  const uint8_t* w;        // W1 codes [L, 2I, H]
  const uint8_t* w_scales; // [L * 2I, ss]
  bf16_t* out;             // h [P, I]
  const int2* tiles;
  const int32_t* num_tiles;
  int32_t H, I, ss;        // ss: scale bytes per row (multiple of 4)
  int32_t* tickets;        // ticket counter of the last rounds (zero at launch), or null
};

__global__ __launch_bounds__(256, 1) void k_gemm_fp8_gate_up(Fp8Args p) {
  constexpr int BM = 256, BN = 256, NW = 4, WN = 2, kThreads = 256;
  constexpr int MS = 8, NS = 8;                    // 16x16 blocks per wave
  constexpr int AL = BM * PPR / kThreads, BL = BN * PPR / kThreads;
  constexpr int NSA = 3;
  __shared__ __attribute__((aligned(16))) uint4 As[NSA][BM * PPR];
  __shared__ __attribute__((aligned(16))) uint4 Bs[2][BN * PPR];
  constexpr uint32_t kStage = BM * PPR * 16, kLoadStride = NW * 1024;
  const int tid = threadIdx.x, wave0 = tid / 64, lane0 = tid % 64;
  const uint32_t swave = (uint32_t)__builtin_amdgcn_readfirstlane(wave0) * 1024u;
  const uint32_t lds_a = (uint32_t)(uintptr_t)&As[0][0] + swave;
  const uint32_t lds_b = (uint32_t)(uintptr_t)&Bs[0][0] + swave;
  const int32_t ntn = (p.I + BN / 2 - 1) / (BN / 2);
  const int32_t nrt = *p.num_tiles;
  const int64_t total = (int64_t)((nrt + GM - 1) / GM) * GM * ntn;
  const int per = gridDim.x / kXcds, xcd = blockIdx.x % kXcds, jx = blockIdx.x / kXcds;
  const int nk = p.H / BKB;
  // Static rounds, except that the items of the last kDynRounds rounds go out by ticket to whichever
  // workgroups ask first (the XCDs do not run at the same speed), shared through a word of a stage
  // buffer that is idle between items.
  const int64_t rounds = (total + gridDim.x - 1) / gridDim.x;
  const int64_t Rs = p.tickets ? max((int64_t)0, rounds - kDynRounds) : rounds;

  for (int64_t round = 0;; ++round) {
    int64_t item = (round * kXcds + xcd) * per + jx;
    if (round >= Rs && p.tickets) {
      int32_t* const word = (int32_t*)&As[2][0];
      if (tid == 0) *word = __hip_atomic_fetch_add(p.tickets, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      item = Rs * gridDim.x + __builtin_amdgcn_readfirstlane(*word);
      __syncthreads();
    }
    if (item >= total) break;
    const int64_t group = item / (GM * ntn), within = item % (GM * ntn);
    const int32_t nt = (int32_t)(within / GM);
    const int32_t mt = (int32_t)(group * GM + within % GM);
    if (mt >= nrt) continue;
    int lane = lane0, wave = wave0;
    asm volatile("" : "+v"(lane), "+v"(wave));
    const int wm = wave / WN, wn = wave % WN;
    const int2 tile = p.tiles[mt];
    const int32_t el = tile.x, m0 = tile.y;
    const int32_t cnt = p.counts[el], eoff = p.offsets[el];  // issued together
    const int32_t valid = min(BM, (int32_t)min((int64_t)cnt, p.clamp) - m0);
    const int32_t off = eoff;
    const int32_t c0 = nt * (BN / 2);
    // W1 row of tile column r (gate rows [0, BN/2), up rows [BN/2, BN); columns past I re-read I-1)
    auto w_row = [&](int r) -> int64_t {
      const int32_t col = min(c0 + (r < BN / 2 ? r : r - BN / 2), p.I - 1);
      return (int64_t)el * 2 * p.I + (r < BN / 2 ? col : p.I + col);
    };
    // per-lane byte offsets (operand rows < 4 GB, checked by the host) of this thread's loads: load
    // i of the wave writes 16-byte slots [(i*NW + wave)*64, +64) of its stage
    // Received rows of this thread's A loads and of its 8 X blocks' scale rows (tile rows past the
    // end re-read the last valid one).  Gathered rows: all 16 loads are issued before any is used.
    const int arow0 = wm * 128 + (lane & 15);
    int32_t ra[AL], rx[MS];
#pragma unroll
    for (int i = 0; i < AL; ++i) ra[i] = min(((i * NW + wave) * 64 + lane) / PPR, valid - 1);
#pragma unroll
    for (int i = 0; i < MS; ++i) rx[i] = min(arow0 + i * 16, valid - 1);
    if (p.perm) {
#pragma unroll
      for (int i = 0; i < AL; ++i) ra[i] = p.perm[off + m0 + ra[i]];
#pragma unroll
      for (int i = 0; i < MS; ++i) rx[i] = p.perm[off + m0 + rx[i]];
#pragma unroll
      for (int i = 0; i < AL; ++i) ra[i] /= p.topk;
#pragma unroll
      for (int i = 0; i < MS; ++i) rx[i] /= p.topk;
    } else {
#pragma unroll
      for (int i = 0; i < AL; ++i) ra[i] += el * (int32_t)p.slab + m0;
#pragma unroll
      for (int i = 0; i < MS; ++i) rx[i] += el * (int32_t)p.slab + m0;
    }
    uint32_t aoff[AL], boff[BL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int slot = (i * NW + wave) * 64 + lane;
      const int r = slot / PPR, c = (slot % PPR) ^ ((r >> 1) & 7);
      aoff[i] = (uint32_t)ra[i] * (uint32_t)p.H + c * 16;
    }
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      const int slot = (i * NW + wave) * 64 + lane;
      const int r = slot / PPR, c = (slot % PPR) ^ ((r >> 1) & 7);
      boff[i] = (uint32_t)(w_row(r) * p.H) + c * 16;
    }
    // scale-row offsets of this lane's 8 X blocks and 8 W blocks (in 32-bit words)
    uint32_t xso[MS], wso[NS];
    // LDS row of W block j for this lane
    auto brow = [&](int j) { return (j < NS / 2 ? 0 : BN / 2) + wn * 64 + (j % (NS / 2)) * 16 + (lane & 15); };
#pragma unroll
    for (int i = 0; i < MS; ++i) xso[i] = (uint32_t)rx[i] * (uint32_t)(p.ss / 4);
#pragma unroll
    for (int j = 0; j < NS; ++j) wso[j] = (uint32_t)(w_row(brow(j)) * p.ss / 4);
    // The scale words are ordinary loads the compiler sees and waits for before their first use, four
    // slices after they are issued.  It does not see the direct-to-LDS loads, so that wait also waits
    // for the stage loads then in flight (those of the next slice, about half a slice early).
    const uint32_t* xsw = (const uint32_t*)p.a_scales;
    const uint32_t* wsw = (const uint32_t*)p.w_scales;

    floatx4_t acc[MS][NS];
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int j = 0; j < NS; ++j) acc[i][j] = floatx4_t{0, 0, 0, 0};

    // A slice is multiplied in two halves over the W blocks (j in [0, 4), then [4, 8)).  wf[h]
    // holds the 4 W fragments of half h; during half 0 the slice's half-1 fragments are read, during
    // half 1 the next slice's half-0 fragments.  X fragments stream along the block rows.
    int8v_t wf[2][NS / 2];
    int8v_t xf[MS];  // this slice's X fragments (slots refilled with the next slice's during half 1)
    uint32_t xs[MS], ws[NS], xsn[MS], wsn[NS];  // scale words of the current / next group of 4 slices
    // Fragment rows step by 16, so the swizzle term ((row >> 1) & 7) is the same for every block of
    // an operand: each lane needs two slot offsets per operand (pieces g and g+4); a block adds
    // 16 rows = 16 * PPR slots.
    const int g = lane >> 4;
    const int xo0 = slot_of_piece(arow0, g), xo1 = slot_of_piece(arow0, g + 4);
    const int wo0 = slot_of_piece(brow(0), g), wo1 = slot_of_piece(brow(0), g + 4);
    auto frag = [](const uint4* stage, int s0, int s1) {
      const uint4 lo = stage[s0];
      const uint4 hi = stage[s1];
      return int8v_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    // X block i / W block j of a stage (W block j sits (brow(j) - brow(0)) rows further)
    auto x_frag = [&](const uint4* stage, int i) { return frag(stage, xo0 + i * 16 * PPR, xo1 + i * 16 * PPR); };
    auto w_frag = [&](const uint4* stage, int j) {
      const int d = ((j < NS / 2 ? 0 : BN / 2) + (j % (NS / 2)) * 16) * PPR;
      return frag(stage, wo0 + d, wo1 + d);
    };
    auto load_scales = [&](int grp, uint32_t (&xd)[MS], uint32_t (&wd)[NS]) {
#pragma unroll
      for (int i = 0; i < MS; ++i) xd[i] = xsw[xso[i] + grp];
#pragma unroll
      for (int j = 0; j < NS; ++j) wd[j] = wsw[wso[j] + grp];
    };
    auto issue_a = [&](int kt, int i) {
      dma16(p.a + (int64_t)kt * BKB, aoff[i], lds_a + (kt % NSA) * kStage + i * kLoadStride);
    };
    auto issue_b = [&](int kt, int i) {
      dma16(p.w + (int64_t)kt * BKB, boff[i], lds_b + (kt & 1) * kStage + i * kLoadStride);
    };
    // the stage loads' waits (vmcnt(0), or all but the newest kCnt loads)
    auto wait_loads = [](auto kWaitAll, auto kCnt) {
      if constexpr (decltype(kWaitAll)::value) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(decltype(kCnt)::value) : "memory");
    };
    auto barrier = [] {
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };

    // prologue: slices 0 and 1 landed; slice 0's half-0 W fragments and first X fragment read
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < AL; ++i) issue_a(0, i);
#pragma unroll
    for (int i = 0; i < BL; ++i) issue_b(0, i);
    if (nk > 1) {
#pragma unroll
      for (int i = 0; i < AL; ++i) issue_a(1, i);
#pragma unroll
      for (int i = 0; i < BL; ++i) issue_b(1, i);
    }
    load_scales(0, xs, ws);
    wait_loads(std::true_type{}, std::integral_constant<int, 0>{});
    barrier();
#pragma unroll
    for (int j = 0; j < NS / 2; ++j) wf[0][j] = w_frag(Bs[0], j);
#pragma unroll
    for (int i = 0; i < MS - 1; ++i) xf[i] = x_frag(As[0], i);

    // Slice kt.  Half 0: A(kt+2) is loaded into the A stage of slice kt-1 (free since the barrier
    // that opened this slice).  Mid barrier: every wave is done with slice kt's W stage; W(kt+1)
    // and A(kt+1) have landed (only the A(kt+2) loads just issued may be pending).  Half 1: the next
    // group's scale words (first slice of a group) and W(kt+2), into slice kt's W stage.
    auto slice = [&]<bool kLoadA, bool kLoadB, bool kNext>(int kt) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      barrier();
      if ((kt & 3) == 0 && kt > 0) {
#pragma unroll
        for (int i = 0; i < MS; ++i) xs[i] = xsn[i];
#pragma unroll
        for (int j = 0; j < NS; ++j) ws[j] = wsn[j];
      }
      const int sh = (kt & 3) * 8;
      const uint4* a_cur = As[kt % NSA];
      const uint4* a_nxt = As[(kt + 1) % NSA];
      const uint4* b_cur = Bs[kt & 1];
      const uint4* b_nxt = Bs[(kt + 1) & 1];
      static_for<2>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        if constexpr (h == 1) {
          // also the scale words of the next group, loaded after a previous slice's mid barrier
          if constexpr (kLoadA) wait_loads(std::false_type{}, std::integral_constant<int, AL>{});
          else wait_loads(std::true_type{}, std::integral_constant<int, 0>{});
          barrier();
          if ((kt & 3) == 0 && kt + 4 < nk) load_scales(kt / 4 + 1, xsn, wsn);
        }
        static_for<MS>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (h == 0 && kLoadA) issue_a(kt + 2, i);
          if constexpr (h == 1 && kLoadB) issue_b(kt + 2, i);
          // X fragments: every block of the slice is read once.  Half 0 reads block 7 (blocks 0-6
          // were read during the previous slice's half 1); half 1 reads the next slice's block i-1
          // into the slot its last use here just freed.
          if constexpr (h == 0 && i == MS - 2) xf[MS - 1] = x_frag(a_cur, MS - 1);
          if constexpr (h == 1 && kNext && i >= 1) xf[i - 1] = x_frag(a_nxt, i - 1);
          // W fragments of the next half: one every other row block
          if constexpr (i % 2 == 1) {
            constexpr int jj = i / 2;
            if constexpr (h == 0) wf[1][jj] = w_frag(b_cur, NS / 2 + jj);
            else if constexpr (kNext) wf[0][jj] = w_frag(b_nxt, jj);
          }
          const int xsc = (int)((xs[i] >> sh) & 0xFFu);
          static_for<NS / 2>([&](auto jc) {
            constexpr int jl = decltype(jc)::value, j = h * (NS / 2) + jl;
            const int wsc = (int)((ws[j] >> sh) & 0xFFu);
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[h][jl], xf[i], acc[i][j], 0, 0, 0, wsc,
                                                                          0, xsc);
          });
        });
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    int kt = 0;
    for (; kt + 2 < nk; ++kt) slice.template operator()<true, true, true>(kt);
    if (kt + 1 < nk) slice.template operator()<false, false, true>(kt++);
    slice.template operator()<false, false, false>(kt);
    // every wave is past its last LDS read before the next item's loads overwrite the stages
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier();

    // Epilogue through LDS, as in the bf16 kernel: each wave packs its 128 x 64 h tile into its own
    // 16 KB of the idle stage buffers (granule g of row r at g ^ (r mod 8)), then stores whole
    // 128-byte row segments, 16 bytes per lane.
    int lane_e = lane, valid_e = valid, off_e = off, m0_e = m0;
    asm volatile("" : "+v"(lane_e), "+v"(valid_e), "+v"(off_e), "+v"(m0_e));
    char* const ot = (char*)(wave < NSA ? &As[wave][0] : &Bs[wave - NSA][0]);
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      const int r = i * 16 + (lane_e & 15);
#pragma unroll
      for (int j = 0; j < NS / 2; ++j) {
        uint2 v;
        v.x = pack_bf16x2(silu_mul(acc[i][j][0], acc[i][j + NS / 2][0]), silu_mul(acc[i][j][1], acc[i][j + NS / 2][1]));
        v.y = pack_bf16x2(silu_mul(acc[i][j][2], acc[i][j + NS / 2][2]), silu_mul(acc[i][j][3], acc[i][j + NS / 2][3]));
        const int g = 2 * j + (lane_e >> 5);
        *(uint2*)(ot + r * 128 + ((g ^ (r & 7)) * 16) + ((lane_e >> 4) & 1) * 8) = v;
      }
    }
    __syncthreads();
    {
      const int g = lane_e % 8;
      const int32_t col = c0 + wn * 64 + g * 8;  // I % 64 == 0: a granule is in or out as a whole
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int r = it * 8 + lane_e / 8;
        const uint4 v = *(const uint4*)(ot + r * 128 + ((g ^ (r & 7)) * 16));
        const int row = wm * 128 + r;
        if (row >= valid_e || col >= p.I) continue;
        *(uint4*)(p.out + (int64_t)(off_e + m0_e + row) * p.I + col) = v;
      }
    }
    __syncthreads();  // the next item's loads reuse the stage buffers
  }
}

int g_cus_fp8[64];

int grid_one_per_cu() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (g_cus_fp8[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cus_fp8[dev] = n;
  }
  const int n = g_cus_fp8[dev] / kXcds * kXcds;
  return n > 0 ? n : kXcds;
}

}  // namespace

hipError_t launch_gemm_gate_up_fp8(const Geom& g, GemmRows rows, const uint8_t* a_codes, const uint8_t* a_scales,
                                   const int32_t* counts, const int32_t* offsets, int64_t count_clamp,
                                   const uint8_t* w_codes, const uint8_t* w_scales, bf16_t* h, const int2* tiles,
                                   const int32_t* num_tiles, hipStream_t stream, int32_t* tickets) {
  Fp8Args a;
  a.a = a_codes;
  a.a_scales = a_scales;
  a.perm = rows.perm;
  a.topk = rows.K;
  a.slab = rows.slab;
  a.counts = counts;
  a.offsets = offsets;
  a.clamp = count_clamp;
  a.w = w_codes;
  a.w_scales = w_scales;
  a.out = h;
  a.tiles = tiles;
  a.num_tiles = num_tiles;
  a.H = g.H;
  a.I = g.I;
  a.ss = fp8_scale_stride(g.H);
  a.tickets = tickets;
  hipLaunchKernelGGL(k_gemm_fp8_gate_up, dim3(grid_one_per_cu()), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
