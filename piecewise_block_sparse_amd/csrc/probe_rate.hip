// Attainable bf16 MFMA rate of gfx950 for the attention kernel's per-chunk
// instruction mix, measured on random operands.
//
// The chip's clock under sustained MFMA work depends on how many operand bits
// toggle: the same instruction stream runs markedly faster on zeros than on
// random data.  The published dense bf16 peak assumes the nominal clock;
// this probe measures what the hardware sustains for the work the exact
// phase of the attention kernel issues, with that kernel's occupancy (three
// 4-wave workgroups per CU, 32-key chunks, d = 128):
//
//   mix = 0  MFMA only: per wave and chunk, S^T = K . Q^T as 8 dependent
//            32x32x16 MFMAs (K from LDS) and O^T += V^T . P^T as 8 MFMAs into
//            four accumulators (V read transposed from LDS); P is S
//            truncated to bf16 (8 byte permutes), no softmax.
//   mix = 1  the full chunk step: the same MFMAs plus the softmax weights
//            (16 exp2, 8 bf16 packs, 8 dot2 sums), a workgroup barrier per
//            chunk and the two-stage global -> LDS copy ring of the next chunk.
//   mix = 2  registers only: the same 16 MFMAs per wave and chunk with every
//            operand in VGPRs (eight A and eight B fragments, cycled so that
//            consecutive MFMAs see different random operands) into four
//            independent accumulators; no LDS, no barrier, no copies.  This
//            separates the clock the chip holds under MFMA work on toggling
//            operands from the cost of feeding the MFMAs from LDS.
//
// Operands: Q in registers, K / V chunks copied from a 2 MB buffer (L2
// resident) of N(0, 1)-like bf16 values; `zeros` = 1 fills everything with
// zeros instead (the same instructions on operands that do not toggle).
//
// pisa_probe_read_rate measures the other roofline the library's streaming
// kernels (statistics, routing) are held to: the HBM read rate of a plain
// streaming reduction over a buffer much larger than the caches.
#include "common.hpp"
#include "lds_stream.hpp"
#include "pisa_probe.h"

namespace pisa {
namespace {

struct ProbeCfg {
  static constexpr int D = 128, RB = 256, CPR = 16, CK = 32;
  static constexpr int NW = 4;
  static constexpr int SUBB = CK * RB;       // 8 KB K (or V) chunk
  static constexpr int STB = 2 * SUBB;       // one ring stage
  static constexpr int DPW = STB / 1024 / NW;
  static constexpr int RPD = 1024 / RB;
  static constexpr int KS = D / 16, MT = D / 32;
};
using PC = ProbeCfg;
constexpr int kWindow = 2 * PC::STB;         // bytes of the source each workgroup streams
constexpr int kWindows = 64;                 // 64 windows: a 2 MB source

__host__ __device__ inline unsigned mix32(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// approximately N(0, 1): sum of four uniforms on [0, 1), centred, times sqrt 3
__device__ inline float normalish(unsigned e) {
  const unsigned h = mix32(e * 2654435761u + 0x9e3779b9u);
  const float s = (float)(h & 255u) + (float)((h >> 8) & 255u) + (float)((h >> 16) & 255u) + (float)(h >> 24);
  return (s / 256.f - 2.f) * 1.7320508f;
}

__device__ inline unsigned pair_at(unsigned e, int zeros) {
  return zeros ? 0u : pack2(normalish(2u * e), normalish(2u * e + 1u));
}

__global__ void fill_kernel(unsigned* p, int n, int zeros) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < n) p[e] = pair_at((unsigned)e, zeros);
}

template <int MIX>
__global__ __launch_bounds__(256, 3) void probe_kernel(const char* src, float* out, int iters, int zeros) {
  __shared__ __attribute__((aligned(1024))) char lds[2 * PC::STB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q32 = lane & 31, hh = lane >> 5;
  const char* win = src + (size_t)(blockIdx.x % kWindows) * kWindow;
  const unsigned m0 = (unsigned)(uintptr_t)(lvoid*)lds;
  const DmaOff<PC> loff = dma_lane_offsets<PC>(w, lane);
  // the attention kernel's two offset bases: every K and V fragment offset is
  // one XOR (and an immediate) away from them
  const int k0 = q32 * PC::RB + ((hh ^ swz<PC::D>(q32)) << 4);
  const int v0 = tr_lane_offset<PC>(lane, 0, 0);
  bf16x8 qf[PC::KS];
#pragma unroll
  for (int ks = 0; ks < PC::KS; ++ks) {
    const unsigned e = 4u * (unsigned)(PC::KS * (blockIdx.x * 256 + tid) + ks) + 0x40000000u;
    qf[ks] = as_bf16x8(u32x4{pair_at(e, zeros), pair_at(e + 1, zeros), pair_at(e + 2, zeros), pair_at(e + 3, zeros)});
  }
  f32x16 acc[PC::MT];
#pragma unroll
  for (int mt = 0; mt < PC::MT; ++mt) acc[mt] = f32x16{};
  float l = 0.f, m = 0.f;
  const float c2 = 0.08838835f * kLog2e;     // 1 / sqrt(128) in log2 units
  const bf16x2 one = {(bf16)1.f, (bf16)1.f};

  dma_stage<PC>(win, win + PC::SUBB, m0, w, loff);
  for (int it = 0; it < iters; ++it) {
    wait_vm0();
    __syncthreads();
    if (it + 1 < iters) {
      const int nx = (it + 1) & 1;
      dma_stage<PC>(win + nx * PC::STB, win + nx * PC::STB + PC::SUBB, m0 + nx * PC::STB, w, loff);
    }
    const char* stage = lds + (it & 1) * PC::STB;
    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < PC::KS; ++ks) s = mfma32(as_bf16x8(ld16(stage + (k0 ^ (32 * ks)))), qf[ks], s);
    u32x4 pf[2];
    if constexpr (MIX) {
      float sum = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float p0 = fast_exp2(fmaf(s[2 * q], c2, -m));
        const float p1 = fast_exp2(fmaf(s[2 * q + 1], c2, -m));
        const bf16x2 pr = {(bf16)p0, (bf16)p1};
        sum = __builtin_amdgcn_fdot2_f32_bf16(pr, one, sum, false);
        pf[q / 4][q % 4] = __builtin_bit_cast(unsigned, pr);
      }
      l += sum;
      if (__any(!(sum < 3.0e38f))) m += 1.f;  // the rescale test of the real loop (not taken)
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q)   // the two logits truncated to bf16, one v_perm each
        pf[q / 4][q % 4] = __builtin_amdgcn_perm(__float_as_uint(s[2 * q + 1]), __float_as_uint(s[2 * q]), 0x07060302u);
      l += s[0];
    }
    const char* vst = stage + PC::SUBB;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
      for (int mt = 0; mt < PC::MT; ++mt)
        acc[mt] = mfma32(as_bf16x8(tr_read<PC>(vst + 8 * PC::RB, sl, (v0 ^ (64 * mt)) - 8 * PC::RB,
                                               (v0 ^ (64 * mt)) ^ 32)),
                         as_bf16x8(pf[sl]), acc[mt]);
  }
  float r = l;
#pragma unroll
  for (int mt = 0; mt < PC::MT; ++mt)
#pragma unroll
    for (int e = 0; e < 16; ++e) r += acc[mt][e];
  out[(size_t)blockIdx.x * 256 + tid] = r;
}

// mix = 2: the MFMA stream alone, operands in registers.  Same grid and
// occupancy as probe_kernel (three 4-wave workgroups per CU).
__global__ __launch_bounds__(256, 3) void probe_regs_kernel(float* out, int iters, int zeros) {
  const int tid = threadIdx.x;
  bf16x8 af[8], bfr[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const unsigned e = 64u * (unsigned)(blockIdx.x * 256 + tid) + 8u * (unsigned)u;
    af[u] = as_bf16x8(u32x4{pair_at(e, zeros), pair_at(e + 1, zeros), pair_at(e + 2, zeros), pair_at(e + 3, zeros)});
    bfr[u] = as_bf16x8(u32x4{pair_at(e + 4, zeros), pair_at(e + 5, zeros), pair_at(e + 6, zeros), pair_at(e + 7, zeros)});
  }
  f32x16 acc[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) acc[a] = f32x16{};
  for (int it = 0; it < iters; ++it) {
    // 16 MFMAs per chunk, as in the exact phase; accumulator a % 4, A fragment
    // u, B fragment (u + 3 (u / 8) + 1) % 8: no two consecutive MFMAs share an operand
#pragma unroll
    for (int u = 0; u < 16; ++u)
      acc[u % 4] = mfma32(af[u % 8], bfr[(u + 3 * (u / 8) + 1) % 8], acc[u % 4]);
  }
  float r = 0.f;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int e = 0; e < 16; ++e) r += acc[a][e];
  out[(size_t)blockIdx.x * 256 + tid] = r;
}

// Streaming read: workgroup b sums words [b * per, (b + 1) * per) of the buffer
// with 16-byte loads, eight per lane in flight; the sum is written only if it
// hits a sentinel, so the loads cannot be dropped.
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                   unsigned* out, int per) {
  constexpr int U = 8;
  const size_t base = (size_t)blockIdx.x * per;
  unsigned acc = 0u;
  for (int i = threadIdx.x; i < per; i += 256 * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t e = base + i + u * 256;
      v[u] = (i + u * 256 < per && e < n16) ? p[e] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] + v[u][1] + v[u][2] + v[u][3];
  }
  if (acc == 0x9e3779b9u) out[blockIdx.x] = acc;
}

}  // namespace
}  // namespace pisa

extern "C" int pisa_probe_read_rate(size_t bytes, int reps, double* gbs) {
  using namespace pisa;
  constexpr int kGrid = 8192;
  if (!gbs || reps < 1 || bytes < (size_t)kGrid * 4096 || bytes % 16 != 0) return (int)hipErrorInvalidValue;
  const size_t n16 = bytes / 16;
  const int per = (int)(n16 / kGrid);
  char* buf = nullptr;
  unsigned* out = nullptr;
  hipEvent_t t0 = nullptr, t1 = nullptr;
  hipError_t e = hipMalloc(&buf, bytes);
  if (e == hipSuccess) e = hipMalloc(&out, kGrid * sizeof(unsigned));
  if (e == hipSuccess) e = hipEventCreate(&t0);
  if (e == hipSuccess) e = hipEventCreate(&t1);
  if (e == hipSuccess) {
    const int nwords = (int)(bytes / 4 < (size_t)INT32_MAX ? bytes / 4 : INT32_MAX);
    fill_kernel<<<(nwords + 255) / 256, 256>>>(reinterpret_cast<unsigned*>(buf), nwords, 0);
    auto launch = [&]() {
      read_kernel<<<kGrid, 256>>>(reinterpret_cast<const u32x4*>(buf), n16, out, per);
    };
    launch();                                // warm-up
    e = hipEventRecord(t0);
    for (int r = 0; r < reps && e == hipSuccess; ++r) launch();
    if (e == hipSuccess) e = hipGetLastError();
    if (e == hipSuccess) e = hipEventRecord(t1);
    if (e == hipSuccess) e = hipEventSynchronize(t1);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t0, t1);
    const double read = (double)per * kGrid * 16.0 * reps;   // bytes the kernels read
    if (e == hipSuccess) *gbs = read / (ms * 1e-3) * 1e-9;
  }
  if (t0) (void)hipEventDestroy(t0);
  if (t1) (void)hipEventDestroy(t1);
  if (out) (void)hipFree(out);
  if (buf) (void)hipFree(buf);
  return (int)e;
}

extern "C" int pisa_probe_chunk_rate(int mix, int zeros, int iters, int reps, double* tflops) {
  using namespace pisa;
  if (!tflops || mix < 0 || mix > 2 || iters < 1 || reps < 1) return (int)hipErrorInvalidValue;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return (int)e;
  const int grid = 3 * cus;
  char* src = nullptr;
  float* out = nullptr;
  hipEvent_t t0 = nullptr, t1 = nullptr;
  const int nwords = kWindows * kWindow / 4;
  e = hipMalloc(&src, (size_t)kWindows * kWindow);
  if (e == hipSuccess) e = hipMalloc(&out, (size_t)grid * 256 * sizeof(float));
  if (e == hipSuccess) e = hipEventCreate(&t0);
  if (e == hipSuccess) e = hipEventCreate(&t1);
  if (e == hipSuccess) {
    fill_kernel<<<(nwords + 255) / 256, 256>>>(reinterpret_cast<unsigned*>(src), nwords, zeros);
    auto launch = [&]() {
      if (mix == 2) probe_regs_kernel<<<grid, 256>>>(out, iters, zeros);
      else if (mix == 1) probe_kernel<1><<<grid, 256>>>(src, out, iters, zeros);
      else probe_kernel<0><<<grid, 256>>>(src, out, iters, zeros);
    };
    launch();                                // warm-up
    e = hipEventRecord(t0);
    for (int r = 0; r < reps && e == hipSuccess; ++r) launch();
    if (e == hipSuccess) e = hipGetLastError();
    if (e == hipSuccess) e = hipEventRecord(t1);
    if (e == hipSuccess) e = hipEventSynchronize(t1);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t0, t1);
    // 16 MFMAs of 32x32x16 (32768 flops) per wave and chunk, 4 waves per workgroup
    const double flops = (double)grid * 4 * iters * 16 * 32768.0 * reps;
    if (e == hipSuccess) *tflops = flops / (ms * 1e-3) * 1e-12;
  }
  if (t0) (void)hipEventDestroy(t0);
  if (t1) (void)hipEventDestroy(t1);
  if (out) (void)hipFree(out);
  if (src) (void)hipFree(src);
  return (int)e;
}
