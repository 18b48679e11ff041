// chip_probe: measured rates of the gfx950 units that bound the attention
// kernels, printed as text.  It is a measurement program beside the library
// (built with it, linked against nothing of it): the roofline figures of the
// prefill are quoted against these numbers next to the specification's peak.
//
//   issue  short single launches (~0.3 ms, before the clock settles): SIMD
//          cycles per wave instruction (launch time x the clock read from the
//          shader clock counter, over the two waves' instructions), for an
//          FMA, an exp2, a 16x16x32 and a 32x32x16 bf16 MFMA, and for one
//          16x16x32 MFMA followed by k independent FMAs (k = 1..4): how much
//          VALU work one MFMA's execution hides.
//   power  20 back-to-back launches (~90 ms) of an MFMA loop on random bf16
//          operands, alone and interleaved with the VALU work the softmax
//          spends per score (an FMA, an exp2, an add and half a bf16 pack per
//          score, 0.5 scores per lane and 16x16x32 MFMA): sustained TFLOP/s
//          and the clock the chip settles at under that power draw; and the
//          bare MFMA loop once more on all-zero operands, whose bits never
//          toggle.
//
//   read   a streaming read of a 4 GiB buffer with 16-byte loads, each
//          workgroup over a contiguous range (plain and non-temporal loads,
//          8 or 16 in flight per lane, workgroups of 512 or 256 lanes, 1 to 4
//          per CU): the HBM read rate the chip delivers to a simple stream,
//          the measured ceiling of the decode, which reads each KV byte once;
//          and the decode's own access pattern (page rows split among the
//          waves of a workgroup, K tiles in the MFMA operand layout) with its
//          arithmetic left out.
//
// With --json only the two 16x16x32 random-operand power rows run (about
// 0.2 s), printed as one JSON object; with --read-json only the streaming
// read (about 0.1 s): the benchmark quotes them next to the specification's
// peaks.
//
// Every workgroup fills one CU (8 waves, two per SIMD; 96 KB of LDS keeps a
// second workgroup off the CU), one workgroup per CU.  The instruction order
// inside each loop is fixed with inline asm (compute instructions only: no
// loads or stores in asm).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;
constexpr size_t kLds = 96 * 1024;

#define CHECK(x)                                                                 \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));             \
      exit(1);                                                                   \
    }                                                                            \
  } while (0)

// Loop bodies.  M16/M32: one MFMA on accumulator i with operand pair
// (ra[i], rb[i + 1]); F, E, A, C: independent VALU chains (FMA, exp2, add,
// bf16 pack).
#define M16(i) asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc[i]) : "v"(ra[i]), "v"(rb[((i) + 1) & 3]))
#define M32(i) \
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc2[i]) : "v"(ra[2 * (i)]), "v"(rb[2 * (i) + 1]))
#define F(i) asm volatile("v_fma_f32 %0, %0, %1, 0.5" : "+v"(fv[i]) : "v"(x))
#define E(i) asm volatile("v_exp_f32 %0, %0" : "+v"(ev[i]))
#define A(i) asm volatile("v_add_f32 %0, %0, %1" : "+v"(sv[i]) : "v"(x))
#define C(i) asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(cv[i]) : "v"(fv[i]), "v"(x))

enum Body {
  kFma16,      // 16 FMAs
  kExp16,      // 16 exp2
  kMfma16,     // 4 x 16x16x32
  kMfma32,     // 2 x 32x32x16 (same FLOPs)
  kMfmaFma1,   // 4 x (16x16x32, 1 FMA)
  kMfmaFma2,   // 4 x (16x16x32, 2 FMA)
  kMfmaFma3,   // 4 x (16x16x32, 3 FMA)
  kMfmaFma4,   // 4 x (16x16x32, 4 FMA)
  kSoft16,     // 4 x 16x16x32 with 2 scores' softmax work (2 FMA, 2 exp2, 2 add, 1 pack)
  kSoft32,     // 2 x 32x32x16 with the same VALU work
  kMfma16Zero, // 4 x 16x16x32 on all-zero operands (no bit toggling)
};

template <int B>
__global__ void __launch_bounds__(kThreads) probe_kernel(const float* in, unsigned long long* out, int iters) {
  const int lane = threadIdx.x & 63;
  const float x = in[lane];
  // pseudo-random bf16 operands (sums of uniforms: roughly normal), four
  // pairs per lane, so that consecutive MFMAs see different data
  bf16x8 ra[4], rb[4];
  const bool zero = B == kMfma16Zero;
  unsigned st = 0x9E3779B9u * (threadIdx.x + 1) + 7919u * blockIdx.x;
  for (int q = 0; q < 4; ++q)
    for (int i = 0; i < 8; ++i) {
      float u = 0.f;
      for (int t = 0; t < 4; ++t) {
        st = st * 1664525u + 1013904223u;
        u += (float)(st >> 8) * (1.0f / 16777216.0f);
      }
      ra[q][i] = (__bf16)(zero ? x : (u - 2.0f) * 1.7f + x);
      st = st * 1664525u + 1013904223u;
      rb[q][i] = (__bf16)(zero ? x : ((float)(st >> 8) * (1.0f / 16777216.0f) - 0.5f) * 3.4f + x);
    }
  f32x4 acc[4] = {};
  f32x16 acc2[2] = {};
  float fv[16], ev[16], sv[4];
  unsigned cv[4];
  for (int j = 0; j < 16; ++j) {
    fv[j] = x + j;
    ev[j] = -x - j;
  }
  for (int j = 0; j < 4; ++j) {
    sv[j] = x;
    cv[j] = j;
  }
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), w0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    if constexpr (B == kFma16) {
      F(0); F(1); F(2); F(3); F(4); F(5); F(6); F(7); F(8); F(9); F(10); F(11); F(12); F(13); F(14); F(15);
    } else if constexpr (B == kExp16) {
      E(0); E(1); E(2); E(3); E(4); E(5); E(6); E(7); E(8); E(9); E(10); E(11); E(12); E(13); E(14); E(15);
    } else if constexpr (B == kMfma16 || B == kMfma16Zero) {
      M16(0); M16(1); M16(2); M16(3);
    } else if constexpr (B == kMfma32) {
      M32(0); M32(1);
    } else if constexpr (B == kMfmaFma1) {
      M16(0); F(0); M16(1); F(1); M16(2); F(2); M16(3); F(3);
    } else if constexpr (B == kMfmaFma2) {
      M16(0); F(0); F(1); M16(1); F(2); F(3); M16(2); F(4); F(5); M16(3); F(6); F(7);
    } else if constexpr (B == kMfmaFma3) {
      M16(0); F(0); F(1); F(2); M16(1); F(3); F(4); F(5); M16(2); F(6); F(7); F(8); M16(3); F(9); F(10); F(11);
    } else if constexpr (B == kMfmaFma4) {
      M16(0); F(0); F(1); F(2); F(3); M16(1); F(4); F(5); F(6); F(7);
      M16(2); F(8); F(9); F(10); F(11); M16(3); F(12); F(13); F(14); F(15);
    } else if constexpr (B == kSoft16) {
      M16(0); F(0); E(0); M16(1); A(0); C(0); M16(2); F(1); E(1); M16(3); A(1);
    } else if constexpr (B == kSoft32) {
      M32(0); F(0); E(0); A(0); M32(1); F(1); E(1); A(1); C(0);
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), w1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  for (int j = 0; j < 16; ++j) s += fv[j] + ev[j];
  for (int j = 0; j < 4; ++j) s += sv[j] + (float)cv[j] + acc[j][0] + acc[j][3];
  for (int k = 0; k < 2; ++k) s += acc2[k][0] + acc2[k][15];
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = t1 - t0;
    out[2 * blockIdx.x + 1] = w1 - w0;
  }
  // never true for the zero input; keeps every result live
  if (in[64 + lane] == 12345.f) out[2 * gridDim.x + threadIdx.x] = (unsigned long long)s;
}

struct Result {
  double ms;         // average per launch
  double clock_ghz;  // shader cycles over real time (100 MHz counter), averaged over workgroups, last launch
};

// Streaming read: workgroup b reads its own contiguous range of 16-byte
// words, U * blockDim words per step (lane t takes words t + j * blockDim of
// the step, U loads in flight), and folds them with xor; the fold is written
// only if it equals a value the buffer's fill cannot give, so the loads stay
// and nothing is written.  words_per_wg is a multiple of U * blockDim.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
template <bool NT, int U>
__global__ void __launch_bounds__(512) read_kernel(const u32x4* src, size_t words_per_wg, unsigned* sink) {
  const u32x4* p = src + (size_t)blockIdx.x * words_per_wg + threadIdx.x;
  const size_t step = (size_t)U * blockDim.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t base = 0; base < words_per_wg; base += step) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const u32x4* q = p + base + (size_t)u * blockDim.x;
      v[u] = NT ? __builtin_nontemporal_load(q) : *q;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9E3779B9u) sink[0] = 1u;
}

struct ReadRow {
  const char* loads;
  int threads, wgs_per_cu, in_flight;
  double gbps;
};

// GB/s of one read configuration over the n-word buffer (10 launches)
template <bool NT, int U>
double time_read(const u32x4* buf, size_t n, unsigned* sink, int n_cu, int threads, int wgs_per_cu) {
  const int wgs = n_cu * wgs_per_cu;
  const size_t step = (size_t)U * threads;
  const size_t words_per_wg = n / wgs / step * step;
  auto k = read_kernel<NT, U>;
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  const int launches = 10;
  hipLaunchKernelGGL(k, dim3(wgs), dim3(threads), 0, 0, buf, words_per_wg, sink);  // warm-up
  CHECK(hipGetLastError());
  CHECK(hipEventRecord(e0));
  for (int r = 0; r < launches; ++r) hipLaunchKernelGGL(k, dim3(wgs), dim3(threads), 0, 0, buf, words_per_wg, sink);
  CHECK(hipGetLastError());
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return (double)words_per_wg * wgs * 16.0 * launches / (ms * 1e-3) / 1e9;
}

// The decode's access pattern without its arithmetic: a pool of 64 KB pages
// (K half: 16 rows of 2 KB, V half likewise), read page after page by 8-wave
// workgroups, wave w taking the 256-byte slice w of every row (one KV head),
// two pages (32 keys, 16 loads per lane) per step.  K tiles: load j of lane
// (r, qd) reads row r, bytes 64 j + 16 qd .. +15 (16 rows x 64 B per
// instruction, the MFMA operand layout); V tiles: row 4 qd + j, bytes 16 r ..
// +15 (4 whole 256-byte rows per instruction).  KPAT_V: the K half read with
// the K pattern as well (half a 128-byte line per row and instruction).
template <bool KPAT_V>
__global__ void __launch_bounds__(512) page_read_kernel(const unsigned char* pool, int pages_per_wg, unsigned* sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, qd = lane >> 4;
  const unsigned char* base = pool + (size_t)blockIdx.x * pages_per_wg * 65536 + 256 * wave;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int pg = 0; pg + 1 < pages_per_wg; pg += 2) {
    u32x4 v[16];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const unsigned char* half = base + (size_t)(pg + t) * 65536 + h * 32768;
        const bool kpat = h == 0 || KPAT_V;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const unsigned char* q = kpat ? half + r * 2048 + 64 * j + 16 * qd : half + (4 * qd + j) * 2048 + 16 * r;
          v[8 * t + 4 * h + j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q));
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) acc ^= v[i];
  }
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9E3779B9u) sink[0] = 1u;
}

// GB/s of the page pattern over the 4 GiB buffer (one 8-wave workgroup per
// CU, 10 launches)
template <bool KPAT_V>
double time_pages(const unsigned char* pool, size_t bytes, unsigned* sink, int n_cu) {
  const int pages_per_wg = (int)(bytes / 65536 / n_cu) & ~1;
  auto k = page_read_kernel<KPAT_V>;
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  const int launches = 10;
  hipLaunchKernelGGL(k, dim3(n_cu), dim3(512), 0, 0, pool, pages_per_wg, sink);  // warm-up
  CHECK(hipGetLastError());
  CHECK(hipEventRecord(e0));
  for (int i = 0; i < launches; ++i) hipLaunchKernelGGL(k, dim3(n_cu), dim3(512), 0, 0, pool, pages_per_wg, sink);
  CHECK(hipGetLastError());
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return (double)n_cu * pages_per_wg * 65536.0 * launches / (ms * 1e-3) / 1e9;
}

constexpr int kReadRows = 16;

// The read rows over a 4 GiB buffer filled with a nonzero pattern: plain and
// non-temporal loads; 8 or 16 loads in flight per lane; workgroups of 512
// lanes (1 or 2 per CU) or 256 lanes (2 or 4 per CU).
int read_rows(int n_cu, ReadRow (&rows)[kReadRows], double (&pages)[2]) {
  const size_t bytes = (size_t)4 << 30, n = bytes / 16;
  u32x4* buf = nullptr;
  unsigned* sink = nullptr;
  if (hipMalloc(&buf, bytes) != hipSuccess) return 1;
  CHECK(hipMalloc(&sink, sizeof(unsigned)));
  CHECK(hipMemsetD32(reinterpret_cast<hipDeviceptr_t>(buf), 0x3C5A7E91, bytes / 4));
  CHECK(hipDeviceSynchronize());
  const int shape[4][2] = {{512, 1}, {512, 2}, {256, 2}, {256, 4}};
  int r = 0;
  for (const auto& sh : shape) {
    rows[r++] = ReadRow{"plain", sh[0], sh[1], 8, time_read<false, 8>(buf, n, sink, n_cu, sh[0], sh[1])};
    rows[r++] = ReadRow{"non-temporal", sh[0], sh[1], 8, time_read<true, 8>(buf, n, sink, n_cu, sh[0], sh[1])};
    rows[r++] = ReadRow{"plain", sh[0], sh[1], 16, time_read<false, 16>(buf, n, sink, n_cu, sh[0], sh[1])};
    rows[r++] = ReadRow{"non-temporal", sh[0], sh[1], 16, time_read<true, 16>(buf, n, sink, n_cu, sh[0], sh[1])};
  }
  const unsigned char* pool = reinterpret_cast<const unsigned char*>(buf);
  pages[0] = time_pages<false>(pool, bytes, sink, n_cu);
  pages[1] = time_pages<true>(pool, bytes, sink, n_cu);
  CHECK(hipFree(buf));
  CHECK(hipFree(sink));
  return 0;
}

template <int B>
Result run(int n_cu, int iters, int launches, const float* in, unsigned long long* d_out, unsigned long long* h_out) {
  auto k = probe_kernel<B>;
  CHECK(hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  hipLaunchKernelGGL(k, dim3(n_cu), dim3(kThreads), kLds, 0, in, d_out, iters);  // warm-up
  CHECK(hipGetLastError());
  CHECK(hipEventRecord(e0));
  for (int r = 0; r < launches; ++r) hipLaunchKernelGGL(k, dim3(n_cu), dim3(kThreads), kLds, 0, in, d_out, iters);
  CHECK(hipGetLastError());
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  CHECK(hipMemcpy(h_out, d_out, sizeof(unsigned long long) * 2 * n_cu, hipMemcpyDeviceToHost));
  double clk = 0.0;
  for (int i = 0; i < n_cu; ++i) clk += (double)h_out[2 * i] / ((double)h_out[2 * i + 1] * 10.0);
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return Result{ms / launches, clk / n_cu};
}

}  // namespace

int main(int argc, char** argv) {
  const bool json = argc > 1 && std::strcmp(argv[1], "--json") == 0;
  const bool read_json = argc > 1 && std::strcmp(argv[1], "--read-json") == 0;
  int dev = 0;
  CHECK(hipSetDevice(dev));
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, dev));
  const int n_cu = prop.multiProcessorCount;
  float* in;
  unsigned long long *d_out, *h_out;
  CHECK(hipMalloc(&in, 128 * sizeof(float)));
  CHECK(hipMemset(in, 0, 128 * sizeof(float)));
  const size_t out_bytes = sizeof(unsigned long long) * (2 * (size_t)n_cu + kThreads);
  CHECK(hipMalloc(&d_out, out_bytes));
  h_out = static_cast<unsigned long long*>(malloc(out_bytes));
  if (!h_out) return 1;
  if (read_json) {
    ReadRow rr[kReadRows];
    double pg[2];
    if (read_rows(n_cu, rr, pg)) return 1;
    int best = 0;
    for (int j = 1; j < kReadRows; ++j)
      if (rr[j].gbps > rr[best].gbps) best = j;
    printf("{\"device\": \"%s\", \"hbm_read_GBps\": %.1f, \"hbm_read_loads\": \"%s\", "
           "\"hbm_read_threads\": %d, \"hbm_read_wgs_per_cu\": %d, \"hbm_read_in_flight\": %d, "
           "\"decode_pattern_GBps\": %.1f, \"buffer_GiB\": 4}\n",
           prop.gcnArchName, rr[best].gbps, rr[best].loads, rr[best].threads, rr[best].wgs_per_cu,
           rr[best].in_flight, pg[0]);
    CHECK(hipFree(in));
    CHECK(hipFree(d_out));
    free(h_out);
    return 0;
  }
  if (json) {
    const int it_long = 65536, launches = 20;
    const double flops = (double)it_long * 4 * (16.0 * 16 * 32 * 2) * n_cu * (kThreads / 64);
    const Result bare = run<kMfma16>(n_cu, it_long, launches, in, d_out, h_out);
    const Result soft = run<kSoft16>(n_cu, it_long, launches, in, d_out, h_out);
    printf("{\"device\": \"%s\", \"mfma_bf16_TFLOPs\": %.1f, \"mfma_bf16_clock_GHz\": %.3f, "
           "\"mfma_bf16_softmax_valu_TFLOPs\": %.1f, \"mfma_bf16_softmax_valu_clock_GHz\": %.3f}\n",
           prop.gcnArchName, flops / (bare.ms * 1e-3) / 1e12, bare.clock_ghz, flops / (soft.ms * 1e-3) / 1e12,
           soft.clock_ghz);
    CHECK(hipFree(in));
    CHECK(hipFree(d_out));
    free(h_out);
    return 0;
  }
  printf("device %s, %d CUs, %d waves per CU (2 per SIMD)\n", prop.gcnArchName, n_cu, kThreads / 64);

  // issue rates: one short launch each; SIMD cycles per loop iteration of one
  // wave = launch cycles / (2 waves x iterations)
  const int it_short = 8192;
  struct Row { const char* name; double instr; Result r; };
  Row rows[] = {
      {"16 x v_fma_f32", 16, run<kFma16>(n_cu, it_short, 1, in, d_out, h_out)},
      {"16 x v_exp_f32", 16, run<kExp16>(n_cu, it_short, 1, in, d_out, h_out)},
      {"4 x mfma 16x16x32 bf16", 4, run<kMfma16>(n_cu, it_short, 1, in, d_out, h_out)},
      {"2 x mfma 32x32x16 bf16", 2, run<kMfma32>(n_cu, it_short, 1, in, d_out, h_out)},
      {"4 x (mfma 16x16x32 + 1 fma)", 4, run<kMfmaFma1>(n_cu, it_short, 1, in, d_out, h_out)},
      {"4 x (mfma 16x16x32 + 2 fma)", 4, run<kMfmaFma2>(n_cu, it_short, 1, in, d_out, h_out)},
      {"4 x (mfma 16x16x32 + 3 fma)", 4, run<kMfmaFma3>(n_cu, it_short, 1, in, d_out, h_out)},
      {"4 x (mfma 16x16x32 + 4 fma)", 4, run<kMfmaFma4>(n_cu, it_short, 1, in, d_out, h_out)},
  };
  printf("\n[issue] short launches (%d iterations per wave, two waves per SIMD)\n", it_short);
  printf("%-30s %14s %14s %10s\n", "loop body", "cycles/iter", "cycles/instr", "clock GHz");
  for (const Row& w : rows) {
    const double per_iter = w.r.ms * 1e6 * w.r.clock_ghz / (2.0 * it_short);
    printf("%-30s %14.2f %14.2f %10.2f\n", w.name, per_iter, per_iter / w.instr, w.r.clock_ghz);
  }

  // sustained: 20 launches of ~4.5 ms each
  const int it_long = 65536, launches = 20;
  const double flops = (double)it_long * 4 * (16.0 * 16 * 32 * 2) * n_cu * (kThreads / 64);
  struct SRow { const char* name; Result r; };
  SRow srows[] = {
      {"mfma 16x16x32 bf16", run<kMfma16>(n_cu, it_long, launches, in, d_out, h_out)},
      {"mfma 32x32x16 bf16", run<kMfma32>(n_cu, it_long, launches, in, d_out, h_out)},
      {"mfma 16x16x32 + softmax VALU", run<kSoft16>(n_cu, it_long, launches, in, d_out, h_out)},
      {"mfma 32x32x16 + softmax VALU", run<kSoft32>(n_cu, it_long, launches, in, d_out, h_out)},
      {"mfma 16x16x32, zero operands", run<kMfma16Zero>(n_cu, it_long, launches, in, d_out, h_out)},
  };
  printf("\n[power] %d back-to-back launches, random bf16 operands (last row: zeros)\n", launches);
  printf("%-30s %12s %14s %10s\n", "loop body", "TFLOP/s", "of 2500 TF/s", "clock GHz");
  for (const SRow& w : srows) {
    const double tf = flops / (w.r.ms * 1e-3) / 1e12;
    printf("%-30s %12.0f %13.1f%% %10.2f\n", w.name, tf, 100.0 * tf / 2500.0, w.r.clock_ghz);
  }

  ReadRow rr[kReadRows];
  double pg[2];
  if (read_rows(n_cu, rr, pg)) return 1;
  printf("\n[read] streaming read of 4 GiB, 16-byte loads, one contiguous range per workgroup, 10 launches\n");
  printf("%-14s %8s %11s %10s %10s %14s\n", "loads", "lanes", "WGs per CU", "in flight", "GB/s", "of 8000 GB/s");
  for (const ReadRow& w : rr)
    printf("%-14s %8d %11d %10d %10.0f %13.1f%%\n", w.loads, w.threads, w.wgs_per_cu, w.in_flight, w.gbps,
           w.gbps / 80.0);
  printf("\n[read] the decode's access pattern without its arithmetic (64 KB pages, 8 waves per CU, non-temporal)\n");
  printf("%-46s %10s %14s\n", "pattern", "GB/s", "of 8000 GB/s");
  printf("%-46s %10.0f %13.1f%%\n", "K tiles 16 rows x 64 B, V tiles 4 rows x 256 B", pg[0], pg[0] / 80.0);
  printf("%-46s %10.0f %13.1f%%\n", "both halves 16 rows x 64 B", pg[1], pg[1] / 80.0);
  CHECK(hipFree(in));
  CHECK(hipFree(d_out));
  free(h_out);
  return 0;
}
