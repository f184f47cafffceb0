// Measured rates of the units the hot path is bound by, on the GPU the library
// runs on: a STREAM-style device copy (the HBM bound of Mean-K build and
// rematerialization), a register-only v_mfma_f32_32x32x16_bf16 loop and a
// v_exp_f32 loop (the two halves of the score passes), and the two together in
// the score passes' own mix: per MFMA, two fused scale-and-shifts, two exps and
// two adds on other registers, so that the loop's score rate is the ceiling the
// instruction mix itself allows when MFMA and VALU work co-issue, measured at
// the score passes' occupancy (two waves per SIMD).
//
// Each measurement launches one untimed and one timed kernel on the given
// stream, times the second with HIP events and waits for it.
#include "common.hpp"

namespace kvm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

static constexpr int PROBE_WG = 2048;        // 8 workgroups of 4 waves per CU
static constexpr int PROBE_WG_MIX = 512;     // 2 per CU: two waves per SIMD, as the score passes
static constexpr int PROBE_THREADS = 256;

// n16 16-byte words from src to dst, one per thread over a grid of one-wave
// workgroups that covers them all, with non-temporal loads and stores: the
// fastest copy shape measured here (medians of 20: 6.68 TB/s for 2 GiB,
// against 6.60 with plain stores, 6.4 with plain loads and stores, 6.1 with
// 256-thread workgroups, 5.6 with four words per thread, 3.6 with sixteen
// loaded before their stores, 4.5-4.9 with grid-stride loops and 4.9-5.0 for
// the runtime's device copy), since the workgroups in flight then cover one
// narrow address range.
static constexpr int PROBE_COPY_TPB = 64;
__global__ __launch_bounds__(PROBE_COPY_TPB) void probe_copy_kernel(const uint4* __restrict__ src,
                                                                    uint4* __restrict__ dst,
                                                                    int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * PROBE_COPY_TPB + threadIdx.x;
  if (i < n16) st_nt(dst + i, ld_nt(src + i));
}

// MODE 0: two MFMA chains; 1: eight exp chains; 2: the score passes' mix.
// Every value ends in `sink` (one float per thread) so nothing is dead code.
template <int MODE>
__global__ __launch_bounds__(256) void probe_alu_kernel(float* __restrict__ sink, int64_t iters) {
  const float t = (float)(threadIdx.x & 63) * 0.015625f;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(t + 0.125f * i);
    b[i] = (__bf16)(0.5f - 0.0625f * i);
  }
  f32x16_t c0 = {}, c1 = {};
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = t - 0.25f * i;
  float acc = 0.0f;
  const float scale = 0.1275f;
  for (int64_t it = 0; it < iters; ++it) {
    if constexpr (MODE == 0) {
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c0) : "v"(a), "v"(b));
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c1) : "v"(a), "v"(b));
    } else if constexpr (MODE == 1) {
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("v_exp_f32 %0, %0" : "+v"(x[i]));
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (h == 0)
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c0) : "v"(a), "v"(b));
        else
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c1) : "v"(a), "v"(b));
        float e0, e1;
        asm volatile(
            "v_fma_f32 %0, %2, %4, -1.0\n"
            "v_fma_f32 %1, %3, %4, -1.0\n"
            "v_exp_f32 %0, %0\n"
            "v_exp_f32 %1, %1\n"
            "s_nop 0\n"
            "v_add_f32 %0, %0, %1"
            : "=&v"(e0), "=&v"(e1)
            : "v"(x[2 * h]), "v"(x[2 * h + 1]), "s"(scale));
        asm volatile("v_add_f32 %0, %0, %1" : "+v"(acc) : "v"(e0));
      }
    }
  }
  float s = acc;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

static int timed(hipStream_t s, hipEvent_t e0, hipEvent_t e1, double* ms,
                 void (*launch)(hipStream_t, void*), void* arg) {
  launch(s, arg);                            // untimed: first-launch costs, clock ramp
  KVM_HIP(hipGetLastError());
  KVM_HIP(hipEventRecord(e0, s));
  launch(s, arg);
  KVM_HIP(hipGetLastError());
  KVM_HIP(hipEventRecord(e1, s));
  KVM_HIP(hipEventSynchronize(e1));
  float f = 0.0f;
  KVM_HIP(hipEventElapsedTime(&f, e0, e1));
  *ms = f;
  return KVM_OK;
}

struct ProbeArgs {
  void* scratch;
  int64_t n;
};

static int measure_rate(int32_t kind, int64_t n, void* scratch, size_t scratch_bytes,
                        double* rate, void* stream) {
  clear_error();
  KVM_CHECK_ARG(rate && scratch, "null pointer");
  KVM_CHECK_ARG(kind >= KVM_RATE_COPY && kind <= KVM_RATE_SCORE_MIX, "unknown rate kind %d", kind);
  KVM_CHECK_ARG(n > 0, "size or iteration count must be positive");
  const size_t sink_bytes = (size_t)PROBE_WG * PROBE_THREADS * sizeof(float);
  if (kind == KVM_RATE_COPY) {
    KVM_CHECK_ARG(n % 16 == 0 && (size_t)n <= scratch_bytes / 2 &&
                      n / 16 / PROBE_COPY_TPB < (1LL << 31),
                  "copy size must be a multiple of 16, at most half the scratch and below 2 TiB");
    KVM_CHECK_ARG((uintptr_t)scratch % 16 == 0, "scratch must be 16-byte aligned");
    KVM_CHECK_RANGE(scratch, (size_t)2 * n, RANGE_DEVICE, "scratch");
  } else {
    KVM_CHECK_ARG(scratch_bytes >= sink_bytes, "scratch needs %zu bytes", sink_bytes);
    KVM_CHECK_RANGE(scratch, sink_bytes, RANGE_DEVICE, "scratch");
  }
  hipStream_t s = as_stream(stream);
  struct Events {            // destroyed on every return
    hipEvent_t e[2] = {nullptr, nullptr};
    ~Events() {
      for (hipEvent_t x : e)
        if (x) (void)hipEventDestroy(x);
    }
  } ev;
  KVM_HIP(hipEventCreate(&ev.e[0]));
  KVM_HIP(hipEventCreate(&ev.e[1]));
  hipEvent_t e0 = ev.e[0], e1 = ev.e[1];
  ProbeArgs pa{scratch, n};
  double ms = 0.0;
  int rc = KVM_OK;
  switch (kind) {
    case KVM_RATE_COPY:
      rc = timed(s, e0, e1, &ms, [](hipStream_t st, void* p) {
        auto* q = static_cast<ProbeArgs*>(p);
        const int64_t n16 = q->n / 16;
        probe_copy_kernel<<<dim3((uint32_t)((n16 + PROBE_COPY_TPB - 1) / PROBE_COPY_TPB)),
                            dim3(PROBE_COPY_TPB), 0, st>>>(
            static_cast<const uint4*>(q->scratch), static_cast<uint4*>(q->scratch) + n16, n16);
      }, &pa);
      if (rc == KVM_OK) *rate = 2.0 * (double)n / (ms * 1e-3);           // bytes read + written
      break;
    case KVM_RATE_MFMA_BF16:
      rc = timed(s, e0, e1, &ms, [](hipStream_t st, void* p) {
        auto* q = static_cast<ProbeArgs*>(p);
        probe_alu_kernel<0><<<dim3(PROBE_WG), dim3(PROBE_THREADS), 0, st>>>(
            static_cast<float*>(q->scratch), q->n);
      }, &pa);
      // 2 MFMAs of 32 x 32 x 16 multiply-adds per iteration and wave
      if (rc == KVM_OK)
        *rate = (double)PROBE_WG * 4 * n * 2 * (2.0 * 32 * 32 * 16) / (ms * 1e-3);
      break;
    case KVM_RATE_EXP:
      rc = timed(s, e0, e1, &ms, [](hipStream_t st, void* p) {
        auto* q = static_cast<ProbeArgs*>(p);
        probe_alu_kernel<1><<<dim3(PROBE_WG), dim3(PROBE_THREADS), 0, st>>>(
            static_cast<float*>(q->scratch), q->n);
      }, &pa);
      if (rc == KVM_OK) *rate = (double)PROBE_WG * PROBE_THREADS * n * 8 / (ms * 1e-3);
      break;
    default:
      rc = timed(s, e0, e1, &ms, [](hipStream_t st, void* p) {
        auto* q = static_cast<ProbeArgs*>(p);
        probe_alu_kernel<2><<<dim3(PROBE_WG_MIX), dim3(PROBE_THREADS), 0, st>>>(
            static_cast<float*>(q->scratch), q->n);
      }, &pa);
      // per MFMA slot a lane takes 2 exps, so a wave 128 score elements
      if (rc == KVM_OK) *rate = (double)PROBE_WG_MIX * 4 * n * 2 * 128 / (ms * 1e-3);
      break;
  }
  return rc;
}

}  // namespace kvm

extern "C" int kvm_measure_rate(int32_t kind, int64_t n, void* scratch, size_t scratch_bytes,
                                double* rate, void* stream) {
  return kvm::guarded([&] { return kvm::measure_rate(kind, n, scratch, scratch_bytes, rate, stream); });
}
