// Exhaustive checks, on the GPU, of the hardware rounding rules the
// quantize-append kernels rely on (test infrastructure: shares no code with
// the library).  Each check compares a rule against a reference computed by
// other means and prints "<name>: mismatches <n>"; a nonzero count fails the
// test that runs this program.
//
//  fp8_e4m3, fp8_e5m2  v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32 on values clamped to
//                      the format's largest finite value, against an encoder
//                      by exponent and mantissa with rintf (round to nearest,
//                      ties to even), for every fp32 bit pattern from 0 to a
//                      little past the largest value and every seventh negative
//  recip_newton        v_rcp_f32 plus one Newton step with FMA, against the
//                      correctly rounded 1.0f / s, for every significand of s
//                      at exponents -40 .. 20
//  div_qmax_<q>        RN(d / q) by the correction step with y = RN(1 / q),
//                      against the correctly rounded division, for every fp32
//                      d in [1e-8, 2^17], q in {3, 15, 127, 255}
//
// Every loop is a bounded grid-stride loop; results go to a small buffer.
#include <hip/hip_runtime.h>
#include <cstdint>
#include <cstdio>
#include <cstring>

namespace {

constexpr float kE4M3Max = 448.0f, kE5M2Max = 57344.0f;

// exponent / mantissa encoders (OCP E4M3FN and E5M2, saturating)
__device__ uint32_t e4m3_by_fields(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), kE4M3Max);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)rintf(a * 512.0f);
  } else {
    int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;
    uint32_t m = (uint32_t)rintf(ldexpf(a, 3 - e));
    if (m == 16) { m = 8; e += 1; }
    code = ((uint32_t)(e + 7) << 3) | (m - 8);
  }
  return code | sign;
}
__device__ uint32_t e5m2_by_fields(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), kE5M2Max);
  uint32_t code;
  if (a < 6.103515625e-05f) {
    code = (uint32_t)rintf(a * 65536.0f);
  } else {
    int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;
    uint32_t m = (uint32_t)rintf(ldexpf(a, 2 - e));
    if (m == 8) { m = 4; e += 1; }
    code = ((uint32_t)(e + 15) << 2) | (m - 4);
  }
  return code | sign;
}

__device__ void record(unsigned long long* cnt, uint32_t* first, uint32_t in, uint32_t got, uint32_t ref) {
  const unsigned long long k = atomicAdd(cnt + 1, 1ull);
  if (k < 4) { first[3 * k] = in; first[3 * k + 1] = got; first[3 * k + 2] = ref; }
}

template <bool E5>
__global__ void fp8_check(uint32_t n, unsigned long long* cnt, uint32_t* first) {
  const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x, nt = gridDim.x * blockDim.x;
  unsigned long long bad = 0;
  for (uint32_t i = tid; i < n; i += nt) {
    for (int sgn = 0; sgn < 2; ++sgn) {
      if (sgn && (i % 7u) != 0) continue;
      const uint32_t bits = i | (sgn ? 0x80000000u : 0u);
      const float x = __uint_as_float(bits);
      const float c = copysignf(fminf(fabsf(x), E5 ? kE5M2Max : kE4M3Max), x);
      const uint32_t hw = E5 ? ((uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c, c, 0, false) & 0xFFu)
                             : ((uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu);
      const uint32_t sw = E5 ? e5m2_by_fields(x) : e4m3_by_fields(x);
      if (hw != sw) { ++bad; record(cnt, first, bits, hw, sw); }
    }
  }
  if (bad) atomicAdd(cnt, bad);
}

__global__ void recip_check(int e_lo, int n_e, unsigned long long* cnt, uint32_t* first) {
  const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x, nt = gridDim.x * blockDim.x;
  const uint32_t n = (uint32_t)n_e << 23;
  unsigned long long bad = 0;
  for (uint32_t i = tid; i < n; i += nt) {
    const uint32_t bits = ((uint32_t)(e_lo + (int)(i >> 23) + 127) << 23) | (i & 0x7FFFFFu);
    const float s = __uint_as_float(bits);
    const float y0 = __builtin_amdgcn_rcpf(s);
    const float er = __builtin_fmaf(-s, y0, 1.0f);
    const float y1 = __builtin_fmaf(er, y0, y0);
    const float ref = 1.0f / s;
    if (__float_as_uint(y1) != __float_as_uint(ref)) { ++bad; record(cnt, first, bits, __float_as_uint(y1), __float_as_uint(ref)); }
  }
  if (bad) atomicAdd(cnt, bad);
}

__global__ void qdiv_check(uint32_t lo_bits, uint32_t n, float q, unsigned long long* cnt, uint32_t* first) {
  const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x, nt = gridDim.x * blockDim.x;
  const float yq = 1.0f / q;
  unsigned long long bad = 0;
  for (uint32_t i = tid; i < n; i += nt) {
    const float d = __uint_as_float(lo_bits + i);
    const float q0 = d * yq;
    const float r = __builtin_fmaf(-q0, q, d);
    const float got = __builtin_fmaf(r, yq, q0);
    const float ref = d / q;
    if (__float_as_uint(got) != __float_as_uint(ref)) { ++bad; record(cnt, first, lo_bits + i, __float_as_uint(got), __float_as_uint(ref)); }
  }
  if (bad) atomicAdd(cnt, bad);
}

bool report(const char* name, unsigned long long* cnt, uint32_t* first) {
  unsigned long long h[2] = {0, 0};
  uint32_t f[12] = {0};
  if (hipDeviceSynchronize() != hipSuccess || hipMemcpy(h, cnt, 16, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(f, first, sizeof f, hipMemcpyDeviceToHost) != hipSuccess) {
    printf("%s: hip error\n", name);
    return false;
  }
  printf("%s: mismatches %llu\n", name, h[0]);
  for (unsigned long long k = 0; k < h[1] && k < 4; ++k) printf("  in 0x%08x got 0x%08x ref 0x%08x\n", f[3 * k], f[3 * k + 1], f[3 * k + 2]);
  return true;
}

}  // namespace

int main() {
  unsigned long long* cnt = nullptr;
  uint32_t* first = nullptr;
  if (hipMalloc(&cnt, 16) != hipSuccess || hipMalloc(&first, 48) != hipSuccess) return 2;
  const dim3 grid(8192), block(256);
  auto reset = [&] { return hipMemset(cnt, 0, 16) == hipSuccess && hipMemset(first, 0, 48) == hipSuccess; };
  bool ok = true;
  float mx;
  uint32_t mb;
  mx = kE4M3Max; memcpy(&mb, &mx, 4);
  ok = ok && reset();
  hipLaunchKernelGGL(fp8_check<false>, grid, block, 0, 0, mb + 0x00100000u, cnt, first);
  ok = ok && report("fp8_e4m3", cnt, first);
  mx = kE5M2Max; memcpy(&mb, &mx, 4);
  ok = ok && reset();
  hipLaunchKernelGGL(fp8_check<true>, grid, block, 0, 0, mb + 0x00100000u, cnt, first);
  ok = ok && report("fp8_e5m2", cnt, first);
  ok = ok && reset();
  hipLaunchKernelGGL(recip_check, grid, block, 0, 0, -40, 61, cnt, first);
  ok = ok && report("recip_newton", cnt, first);
  const float lo = 1e-8f, hi = 131072.0f;
  uint32_t lb, hb;
  memcpy(&lb, &lo, 4);
  memcpy(&hb, &hi, 4);
  const float qs[4] = {3.0f, 15.0f, 127.0f, 255.0f};
  for (float q : qs) {
    ok = ok && reset();
    hipLaunchKernelGGL(qdiv_check, grid, block, 0, 0, lb, hb - lb + 1, q, cnt, first);
    char name[32];
    snprintf(name, sizeof name, "div_qmax_%d", (int)q);
    ok = ok && report(name, cnt, first);
  }
  (void)hipFree(cnt);
  (void)hipFree(first);
  return ok ? 0 : 3;
}
