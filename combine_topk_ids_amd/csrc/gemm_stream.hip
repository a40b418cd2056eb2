// Weight-streaming down GEMM for experts with few rows (decode-sized), bf16 MFMA with fp32
// accumulation: the same product as the down GEMM in gemm.hip (FlashInfer "MoE-EP implementation
// & usage", section 2 "Call stack"; w2 [E, H, I], section 4),  y = h W2_e^T,  over the 64-row
// expert tiles of the device-built tile table.
//
// With a few dozen rows per expert the GEMM is bound by reading W2 once from HBM.  Streaming a
// weight panel 128 bytes of each row at a time (the 64x256 kernel's k-slices) reaches about
// 5.0 TB/s when the rows are 4 KB apart (I = 2048), against 6.1 TB/s when each row gives 512
// contiguous bytes per slice (a copy-only probe of both patterns through LDS, same bytes in
// flight).  This kernel therefore takes k-stages of 256 (512 bytes of every A and W row), 64 W rows
// (output columns) per item, two stages of 32 KB + 32 KB in LDS (one workgroup per CU).  A tile of
// at most 32 rows loads only those 32 A rows, in three stages of 16 KB + 32 KB, so that two stages
// of W are in flight while one is read.
// LDS rows are 32 pieces of 16 bytes, piece c of row r at slot 32r + (c ^ (r & 31)), so the
// 16-byte fragment reads of 32 rows are conflict-free and each direct-to-LDS load instruction
// fetches two whole 512-byte row segments.  Two waves of 32x32 MFMA blocks; the weight fragment is
// the MFMA's first operand, so a lane's accumulators hold four consecutive output columns of one
// row (8-byte stores).
#include "gemm_stream.h"

namespace moe {
namespace {

constexpr int kBM = 64;                     // rows per tile (the tile table's height)
constexpr int kWR = 64;                     // W rows per item
constexpr int kBKS = 256;                   // k per stage
constexpr int kPPR = kBKS / 8;              // 16-byte pieces per LDS row
constexpr int kNW = 2;                      // waves
constexpr int kThreads = kNW * 64;
constexpr int kSlots = kBM * kPPR;          // 16-byte slots per stage and operand (kWR == kBM)
constexpr int kLoads = kSlots / kThreads;   // direct-to-LDS loads per thread, operand and stage
static_assert(kWR == kBM, "A and W stages have the same shape");

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// lane l's 16 bytes from src land at LDS byte lds_byte + 16*l (lds_byte wave-uniform); m0 is
// clobbered and used by nothing else here
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_byte), "v"(src) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ int sslot(int r, int c) { return r * kPPR + (c ^ (r & 31)); }

__device__ __forceinline__ floatx16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const floatx16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS: one ring of k-stages, each kAR A rows then kWR W rows of 512 bytes.  kAR == 64: two stages
// of 64 KB; kAR == 32: three of 48 KB (stages ks+1 and ks+2 in flight while stage ks is read).
constexpr int kLdsBytes = 3 * (32 + kWR) * kPPR * 16;
static_assert(kLdsBytes >= 2 * (64 + kWR) * kPPR * 16, "both rings fit");

// The k-loop of one item over kAR A rows (64, or 32 when the tile has at most 32 rows: half the A
// bytes per stage and a third stage in flight).  kAR == 64: wave w takes A rows 32w.. against both
// 32-row W blocks; kAR == 32: both waves take the 32 A rows, wave w against W block w.
template <int kAR>
__device__ __forceinline__ void stream_k_loop(const bf16_t* const (&asrc)[kLoads], const bf16_t* const (&wsrc)[kLoads],
                                              uint32_t lds_wave, const uint4* lds, int nks, int rot, int lane,
                                              int wave, floatx16_t (&acc)[2]) {
  constexpr int kAL = kAR * kPPR / kThreads;         // A loads per thread and stage
  constexpr int kNS = kAR == 32 ? 3 : 2;             // stages in the ring
  constexpr int kASlots = kAR * kPPR, kStageSlots = kASlots + kSlots;
  constexpr uint32_t kStage = kStageSlots * 16, kLoadStride = kNW * 1024;
  // k-stage ks of the loop holds k-stage (ks + rot) mod nks of the rows
  auto issue = [&](int ks, int buf) {
    ks += rot;
    if (ks >= nks) ks -= nks;
    const uint32_t st = lds_wave + buf * kStage;
#pragma unroll
    for (int i = 0; i < kAL; ++i) dma16(asrc[i] + (int64_t)ks * kBKS, st + i * kLoadStride);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) dma16(wsrc[i] + (int64_t)ks * kBKS, st + kASlots * 16 + i * kLoadStride);
  };
  const int ar = (kAR == 64 ? wave * 32 : 0) + (lane & 31);
  // every wave is done with the previous item's stages (the barrier ending its k-loop)
#pragma unroll
  for (int j = 0; j < kNS - 1; ++j)
    if (j < nks) issue(j, j);
  int buf = 0;
  for (int ks = 0; ks < nks; ++ks) {
    // stage ks+kNS-1 goes into the stage every wave finished reading at the previous barrier; then
    // stage ks must have landed (only the later stages' loads may still be in flight)
    const int ahead = min(nks - 1 - ks, kNS - 1);  // stages issued after stage ks
    if (ks + kNS - 1 < nks) issue(ks + kNS - 1, buf == 0 ? kNS - 1 : buf - 1);
    if (kNS == 3 && ahead == 2) asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * (kAL + kLoads)) : "memory");
    else if (ahead >= 1) asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kAL + kLoads) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    const uint4* a_s = lds + buf * kStageSlots;
    const uint4* w_s = a_s + kASlots;
#pragma unroll
    for (int step = 0; step < kBKS / 16; ++step) {
      const int c = step * 2 + (lane >> 5);
      const bf16x8_t xa = *(const bf16x8_t*)&a_s[sslot(ar, c)];
      if constexpr (kAR == 64) {
        const bf16x8_t xb0 = *(const bf16x8_t*)&w_s[sslot(lane & 31, c)];
        const bf16x8_t xb1 = *(const bf16x8_t*)&w_s[sslot(32 + (lane & 31), c)];
        acc[0] = mfma32(xb0, xa, acc[0]);
        acc[1] = mfma32(xb1, xa, acc[1]);
      } else {
        const bf16x8_t xb = *(const bf16x8_t*)&w_s[sslot(wave * 32 + (lane & 31), c)];
        acc[0] = mfma32(xb, xa, acc[0]);
      }
    }
    // every wave is past its reads of this stage before it is refilled
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    buf = buf == kNS - 1 ? 0 : buf + 1;
  }
}

// down GEMM: y rows = h rows W2^T over 64-row tiles and 64-column items
__global__ __launch_bounds__(kThreads, 1) void k_gemm_stream_down(StreamArgs p) {
  __shared__ __attribute__((aligned(16))) uint4 lds[kLdsBytes / 16];
  const int tid = threadIdx.x, wave0 = tid / 64, lane0 = tid % 64;
  const uint32_t swave = (uint32_t)__builtin_amdgcn_readfirstlane(wave0) * 1024u;
  const uint32_t lds_wave = (uint32_t)(uintptr_t)&lds[0] + swave;
  const int32_t ntn = (p.H + kWR - 1) / kWR;
  const int64_t total = (int64_t)*p.num_tiles * ntn;
  const int nks = p.Kd / kBKS;

  for (int64_t item = blockIdx.x; item < total; item += gridDim.x) {
    const int32_t mt = (int32_t)(item / ntn), nt = (int32_t)(item % ntn);
    // per-thread index values re-derived per item (no hoisting of their addresses)
    int lane = lane0, wave = wave0;
    asm volatile("" : "+v"(lane), "+v"(wave));
    const int2 tile = p.tiles[mt];
    const int32_t el = tile.x, m0 = tile.y;
    const int32_t cnt = p.counts[el], eoff = p.offsets[el];  // issued together
    const int32_t valid = min(kBM, (int32_t)min((int64_t)cnt, p.clamp) - m0);
    const int32_t off = eoff;
    const int32_t c0 = nt * kWR;

    // This thread's loads: load i of the wave fills slots [(i*kNW + wave)*64, +64) of a stage, two
    // rows' 512-byte segments.  A rows past the tile and W rows past the last column re-read a
    // valid row (never stored).
    const bf16_t* asrc[kLoads];
    const bf16_t* wsrc[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int slot = (i * kNW + wave) * 64 + lane;
      const int r = slot / kPPR, c = (slot % kPPR) ^ (r & 31);
      asrc[i] = p.a + ((int64_t)off + m0 + min(r, valid - 1)) * p.Kd + c * 8;
      wsrc[i] = p.w + ((int64_t)el * p.H + min(c0 + r, p.H - 1)) * p.Kd + c * 8;
    }

    floatx16_t acc[2];
    acc[0] = floatx16_t{0};
    acc[1] = floatx16_t{0};
    const bool half = valid <= 32;  // uniform over the workgroup
    // Items take their k-stages in rotated order, starting at stage (item / 8) mod nks, so that the
    // workgroups in flight read different k offsets of their rows.  With I = 2048 the rows are 4 KB
    // apart, and all workgroups reading the same 512-byte column of their rows at once measured 3.4%
    // slower (decode down 193.0 -> 186.5 us; starting at item mod nks, the same stage for every
    // workgroup of an XCD under the round-robin dispatch: 187.6 us).
    const int rot = (int)((item >> 3) % nks);
    if (half) stream_k_loop<32>(asrc, wsrc, lds_wave, lds, nks, rot, lane, wave, acc);
    else stream_k_loop<64>(asrc, wsrc, lds_wave, lds, nks, rot, lane, wave, acc);

    // Epilogue: lane l holds output row l % 32 of its A rows and, in registers 4g..4g+3, the four
    // consecutive output columns 8g + 4(l/32) + 0..3 of a 32-column W block.
    const int row = (half ? 0 : wave * 32) + (lane & 31);
    if (row < valid) {
      const int64_t orow = p.out_slab ? (int64_t)el * p.out_slab + m0 + row : (int64_t)off + m0 + row;
      bf16_t* dst = p.out + orow * p.H;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (half && j == 1) break;
        const int32_t blk = half ? wave : j;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int32_t col = c0 + blk * 32 + 8 * g + 4 * (lane >> 5);
          if (col >= p.H) continue;  // H % 128 == 0
          uint2 v;
          v.x = pack_bf16x2(acc[j][4 * g + 0], acc[j][4 * g + 1]);
          v.y = pack_bf16x2(acc[j][4 * g + 2], acc[j][4 * g + 3]);
          *(uint2*)(dst + col) = v;
        }
      }
    }
  }
}

int g_cus_stream[64];

int grid_one_per_cu_stream() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (g_cus_stream[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cus_stream[dev] = n;
  }
  return g_cus_stream[dev];
}

}  // namespace

bool gemm_stream_fits(int32_t Kd) { return Kd > 0 && Kd % kBKS == 0; }

hipError_t launch_gemm_stream_down(const StreamArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(k_gemm_stream_down, dim3(grid_one_per_cu_stream()), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
