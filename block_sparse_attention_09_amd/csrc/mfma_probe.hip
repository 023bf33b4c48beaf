// What one MI355X sustains on the instruction mixes the attention kernel is
// made of: chains of 32x32x16 fp16/bf16 MFMAs alone, and the same chains with
// independent vector FMAs or exponentials issued between them from the same
// wave.  A measurement program (not part of libabatt): it prints one JSON
// line per case with the time and the MFMA rate.
//
// Each wave runs 8 independent accumulator chains (no chain waits on its own
// previous MFMA) for `iters` rounds; operands are random bits read once from
// device memory.  Work-groups of 4 waves, one (or two) work-groups per CU, so
// one (or two) waves per SIMD.  Only memory access: the operand read and one
// store per thread of a checksum, both inside the buffers allocated below.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChains = 8;

// MODE: 0 fp16 MFMA, 1 bf16 MFMA; EXTRA: 0 none, 1 FMA, 2 exp; NX: extra ops per MFMA
template <int MODE, int EXTRA, int NX>
__global__ __launch_bounds__(256) void probe(const uint32_t* __restrict__ bits,
                                             float* __restrict__ out, int iters) {
  const int gid = blockIdx.x * 256 + threadIdx.x;
  f16x8 a, b;
  {
    const uint32_t* p = bits + (size_t)gid * 8;
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = p[i] & 0x3bff3bffu;  // finite, |x| < 1 in both formats
    a = __builtin_bit_cast(f16x8, (uint32_t __attribute__((ext_vector_type(4)))){w[0], w[1], w[2], w[3]});
    b = __builtin_bit_cast(f16x8, (uint32_t __attribute__((ext_vector_type(4)))){w[4], w[5], w[6], w[7]});
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = 0.5f + 0.01f * (float)((gid + i) & 7);
  const float y = 0.999f;
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      if constexpr (MODE == 0)
        asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(acc[c]) : "v"(a), "v"(b));
      else
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc[c]) : "v"(a), "v"(b));
#pragma unroll
      for (int k = 0; k < NX; ++k) {
        if constexpr (EXTRA == 1)
          asm volatile("v_fma_f32 %0, %0, %1, 0.5" : "+v"(x[k & 7]) : "v"(y));
        else if constexpr (EXTRA == 2)
          asm volatile("v_exp_f32_e64 %0, -%0" : "+v"(x[k & 7]));   // x = 2^-x stays in (0.5, 1)
      }
    }
  }
  // wait states before the accumulators are read by vector instructions
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  out[gid] = s;
}

template <int MODE, int EXTRA, int NX>
static void run(const char* name, const uint32_t* bits, float* out, int cus, int waves, int iters) {
  const int grid = cus * waves;
  hipEvent_t e0, e1;
  hipEventCreate(&e0);
  hipEventCreate(&e1);
  probe<MODE, EXTRA, NX><<<grid, 256>>>(bits, out, iters);   // warm-up (clock ramp)
  probe<MODE, EXTRA, NX><<<grid, 256>>>(bits, out, iters);
  hipEventRecord(e0);
  const int reps = 3;
  for (int r = 0; r < reps; ++r) probe<MODE, EXTRA, NX><<<grid, 256>>>(bits, out, iters);
  hipEventRecord(e1);
  hipEventSynchronize(e1);
  float ms = 0.f;
  hipEventElapsedTime(&ms, e0, e1);
  ms /= reps;
  const double mfma = (double)grid * 4 * iters * kChains;     // per launch
  const double tflops = mfma * 32.0 * 32.0 * 16.0 * 2.0 / (ms * 1e-3) / 1e12;
  std::printf("{\"case\": \"%s\", \"waves_per_simd\": %d, \"extra_per_mfma\": %d, \"ms\": %.4f, "
              "\"mfma_tflops\": %.1f, \"frac_of_2500\": %.3f}\n",
              name, waves, NX, ms, tflops, tflops / 2500.0);
  std::fflush(stdout);
  hipEventDestroy(e0);
  hipEventDestroy(e1);
}

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 4000;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, 0) != hipSuccess) return 1;
  const int cus = prop.multiProcessorCount;
  const size_t threads = (size_t)cus * 2 * 256;
  uint32_t* bits = nullptr;
  float* out = nullptr;
  if (hipMalloc(&bits, threads * 8 * sizeof(uint32_t)) != hipSuccess) return 1;
  if (hipMalloc(&out, threads * sizeof(float)) != hipSuccess) return 1;
  {
    std::vector<uint32_t> h(threads * 8);
    uint64_t s = 0x9E3779B97F4A7C15ull;
    for (auto& v : h) {  // xorshift64*: random operand bits
      s ^= s >> 12;
      s ^= s << 25;
      s ^= s >> 27;
      v = (uint32_t)((s * 0x2545F4914F6CDD1Dull) >> 32);
    }
    if (hipMemcpy(bits, h.data(), h.size() * sizeof(uint32_t), hipMemcpyHostToDevice) != hipSuccess)
      return 1;
  }
  std::printf("{\"device\": \"%s\", \"cus\": %d, \"iters\": %d}\n", prop.name, cus, iters);
  for (int waves = 1; waves <= 2; ++waves) {
    run<0, 0, 0>("mfma_f16", bits, out, cus, waves, iters);
    run<1, 0, 0>("mfma_bf16", bits, out, cus, waves, iters);
    run<0, 1, 4>("mfma_f16+fma", bits, out, cus, waves, iters);
    run<0, 1, 6>("mfma_f16+fma", bits, out, cus, waves, iters);
    run<0, 1, 8>("mfma_f16+fma", bits, out, cus, waves, iters);
    run<0, 2, 1>("mfma_f16+exp", bits, out, cus, waves, iters);
    run<0, 2, 2>("mfma_f16+exp", bits, out, cus, waves, iters);
    run<0, 2, 4>("mfma_f16+exp", bits, out, cus, waves, iters);
  }
  hipFree(bits);
  hipFree(out);
  return 0;
}
