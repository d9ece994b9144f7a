// Calibration micro-benchmarks (see sa_probes.h): MFMA issue rate and shader
// clock, VALU FMA and exp rates, LDS read instruction rates, fp32 atomic-add
// throughput.  Every kernel works on registers or on in-bounds buffers and
// runs a fixed number of iterations.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_probes.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

constexpr int kBlocks = 1024, kThreads = 256;  // 4096 waves: 4 per SIMD on 256 CUs

// Four independent accumulator chains per wave; clock stamps from lane 0 of
// workgroup 0 (cycle counter and the 100 MHz real-time counter).
__global__ __launch_bounds__(kThreads) void k_mfma(float* sink, uint64_t* stamps, int iters) {
  const float f = float(threadIdx.x & 7) * 0.001f;
  bf16x8 a, b;
  for (int j = 0; j < 8; ++j) {
    a[j] = __bf16(f + j);
    b[j] = __bf16(f - j);
  }
  floatx16 acc[4];
  for (int j = 0; j < 4; ++j) acc[j] = floatx16{};
  uint64_t c0 = 0, r0 = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    c0 = __builtin_readcyclecounter();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
  for (int j = 0; j < 4; ++j)
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    stamps[0] = __builtin_readcyclecounter() - c0;
    stamps[1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
  if (s == 1234.5f) sink[threadIdx.x] = s;  // keeps the loop; never true for these inputs
}

template <bool EXP>
__global__ __launch_bounds__(kThreads) void k_valu(float* sink, int iters) {
  float x[8];
  for (int j = 0; j < 8; ++j) x[j] = float(threadIdx.x + j) * 1e-7f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = EXP ? __builtin_amdgcn_exp2f(x[j]) : fmaf(x[j], 0.999f, 1e-7f);
  }
  float s = 0.f;
  for (int j = 0; j < 8; ++j) s += x[j];
  if (s == -1.0f) sink[threadIdx.x] = s;
}

// LDS reads: each wave reads 16 bytes (or 8 bytes transposed) per lane from a
// 16 KB tile at a rotating offset, XOR-folding the data so the reads stay live.
template <bool TR>
__global__ __launch_bounds__(kThreads) void k_lds(int* sink, int iters) {
  __shared__ __attribute__((aligned(16))) short tile[8192];  // 16 KB
  for (int i = threadIdx.x; i < 8192; i += kThreads) tile[i] = short(i);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  int acc = 0;
  for (int i = 0; i < iters; ++i) {
    const int base = ((i * 1024) & 8191) & ~511;  // element offset, 1 KB steps, wraps inside the tile
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int off = (base + j * 64 + lane * 8) & 8191;  // 8 shorts = 16 bytes per lane
      if (TR) {
        const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16*)((__attribute__((address_space(3))) short*)(tile + (off & ~3))));
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
      } else {
        const int4 v = *reinterpret_cast<const int4*>(&tile[off]);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
      }
    }
  }
  if (acc == 0x7fffffff) sink[threadIdx.x] = acc;
}

__device__ __forceinline__ uint32_t hash32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

// 32 KB row blocks (8192 floats) of a buffer of nblocks blocks, chosen by a hash.
template <bool ATOMIC>
__global__ __launch_bounds__(kThreads) void k_update(float* buf, int nblocks, int iters) {
  for (int r = 0; r < iters; ++r) {
    const int rb = int(hash32(uint32_t(blockIdx.x) * 977u + uint32_t(r) * 131u) % uint32_t(nblocks));
    float* base = buf + size_t(rb) * 8192;
#pragma unroll 8
    for (int j = 0; j < 32; ++j) {
      if (ATOMIC) unsafeAtomicAdd(base + j * kThreads + threadIdx.x, 1.0f);
      else base[j * kThreads + threadIdx.x] = 1.0f;
    }
  }
}

#define PCHECK(x)                    \
  do {                               \
    if ((x) != hipSuccess) {         \
      (void)hipGetLastError();       \
      rc = -4;                       \
      goto done;                     \
    }                                \
  } while (0)

template <typename F>
hipError_t time_ms(hipEvent_t a, hipEvent_t b, float* ms, F launch) {
  launch();  // warm-up
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return e;
  float best = 1e30f;
  for (int rep = 0; rep < 3; ++rep) {
    if ((e = hipEventRecord(a, 0)) != hipSuccess) return e;
    launch();
    if ((e = hipEventRecord(b, 0)) != hipSuccess) return e;
    if ((e = hipEventSynchronize(b)) != hipSuccess) return e;
    float t = 0.f;
    if ((e = hipEventElapsedTime(&t, a, b)) != hipSuccess) return e;
    best = t < best ? t : best;
  }
  *ms = best;
  return hipGetLastError();
}

}  // namespace

extern "C" int sa_probe_run(sa_probe_results* out) {
  if (!out) return -1;
  int rc = 0;
  float* sink = nullptr;
  float* buf = nullptr;
  uint64_t* stamps = nullptr;
  hipEvent_t a = nullptr, b = nullptr;
  const int nblocks = 1536;  // 50 MB of 32 KB blocks
  float ms = 0.f;
  uint64_t st[2] = {0, 0};
  const int mfma_iters = 2000, valu_iters = 4000, lds_iters = 2000, upd_iters = 16;
  PCHECK(hipMalloc(&sink, kThreads * sizeof(float)));
  PCHECK(hipMalloc(&stamps, 2 * sizeof(uint64_t)));
  PCHECK(hipMalloc(&buf, size_t(nblocks) * 8192 * sizeof(float)));
  PCHECK(hipMemset(buf, 0, size_t(nblocks) * 8192 * sizeof(float)));
  PCHECK(hipEventCreate(&a));
  PCHECK(hipEventCreate(&b));
  {
    const double waves = double(kBlocks) * kThreads / 64;
    const double simds = 256.0 * 4;
    PCHECK(time_ms(a, b, &ms, [&] { hipLaunchKernelGGL(k_mfma, dim3(kBlocks), dim3(kThreads), 0, 0, sink, stamps, mfma_iters); }));
    PCHECK(hipMemcpy(st, stamps, sizeof(st), hipMemcpyDeviceToHost));
    const double mfmas = waves * mfma_iters * 4;
    out->mfma_bf16_tflops = mfmas * 32768.0 / (ms * 1e-3) / 1e12;
    out->shader_clock_ghz = st[1] ? double(st[0]) / (double(st[1]) * 10.0) : 0.0;  // 100 MHz real-time clock
    const double cycles = ms * 1e-3 * out->shader_clock_ghz * 1e9;
    out->mfma_cycles = cycles * simds / mfmas;
    PCHECK(time_ms(a, b, &ms, [&] { hipLaunchKernelGGL(k_valu<false>, dim3(kBlocks), dim3(kThreads), 0, 0, sink, valu_iters); }));
    out->fma_cycles = ms * 1e-3 * out->shader_clock_ghz * 1e9 * simds / (waves * valu_iters * 8);
    PCHECK(time_ms(a, b, &ms, [&] { hipLaunchKernelGGL(k_valu<true>, dim3(kBlocks), dim3(kThreads), 0, 0, sink, valu_iters); }));
    out->exp_cycles = ms * 1e-3 * out->shader_clock_ghz * 1e9 * simds / (waves * valu_iters * 8);
    PCHECK(time_ms(a, b, &ms, [&] { hipLaunchKernelGGL(k_lds<false>, dim3(kBlocks), dim3(kThreads), 0, 0, reinterpret_cast<int*>(sink), lds_iters); }));
    out->lds_b128_cycles = ms * 1e-3 * out->shader_clock_ghz * 1e9 * 256.0 / (waves * lds_iters * 8);
    PCHECK(time_ms(a, b, &ms, [&] { hipLaunchKernelGGL(k_lds<true>, dim3(kBlocks), dim3(kThreads), 0, 0, reinterpret_cast<int*>(sink), lds_iters); }));
    out->lds_tr_b64_cycles = ms * 1e-3 * out->shader_clock_ghz * 1e9 * 256.0 / (waves * lds_iters * 8);
    const double bytes = double(4096) * upd_iters * 8192 * 4;
    PCHECK(time_ms(a, b, &ms, [&] { hipLaunchKernelGGL(k_update<true>, dim3(4096), dim3(kThreads), 0, 0, buf, nblocks, upd_iters); }));
    out->atomic_f32_tbs = bytes / (ms * 1e-3) / 1e12;
    PCHECK(time_ms(a, b, &ms, [&] { hipLaunchKernelGGL(k_update<false>, dim3(4096), dim3(kThreads), 0, 0, buf, nblocks, upd_iters); }));
    out->store_f32_tbs = bytes / (ms * 1e-3) / 1e12;
  }
done:
  if (a) (void)hipEventDestroy(a);
  if (b) (void)hipEventDestroy(b);
  if (sink) (void)hipFree(sink);
  if (stamps) (void)hipFree(stamps);
  if (buf) (void)hipFree(buf);
  return rc;
}
