// valu_rate.hip -- issue rate of single fp32 VALU operations on one MI355X (gfx950), used to
// set the compositing kernels' arithmetic ceiling.  Each lane runs 8 independent chains of
// one operation (fma, mul, add, exp2, rcp, sqrt, log2, DPP row-shift move) over 8192
// workgroups of 256 lanes, timed with HIP events; prints lane-operations per second.
// Build and run (from the repository root):
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//     tile_differentiable_rasterizer_amd/measure/valu_rate.hip -o /tmp/valu_rate && /tmp/valu_rate
#include <hip/hip_runtime.h>
#include <cstdio>
constexpr int kIters = 4096;
template <int OP>
__global__ __launch_bounds__(256) void k(float* out, float seed) {
  float x[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) x[c] = seed + 0.01f * c + 1e-7f * threadIdx.x;
  for (int i = 0; i < kIters; ++i) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if (OP == 0) x[c] = __builtin_fmaf(x[c], 0.999f, 0.001f);
      if (OP == 1) x[c] = __builtin_amdgcn_exp2f(x[c]);
      if (OP == 2) x[c] = __builtin_amdgcn_rcpf(x[c]);
      if (OP == 3) x[c] = __builtin_amdgcn_sqrtf(x[c]);
      if (OP == 4) x[c] = __builtin_amdgcn_logf(x[c]);
      if (OP == 5) x[c] = x[c] * 0.999f;
      if (OP == 6) x[c] = x[c] + 0.001f;
      if (OP == 9) x[c] = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x[c]), 0x111, 0xF, 0xF, false));
      if (OP == 10) x[c] = __builtin_fmaf(x[c], x[(c + 1) & 7], 0.001f);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) s += x[c];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}
template <int OP>
void run(const char* name, float* out, int blocks) {
  hipEvent_t a, b; (void)hipEventCreate(&a); (void)hipEventCreate(&b);
  k<OP><<<blocks, 256>>>(out, 0.5f);
  (void)hipEventRecord(a);
  for (int r = 0; r < 5; ++r) k<OP><<<blocks, 256>>>(out, 0.5f);
  (void)hipEventRecord(b); (void)hipEventSynchronize(b);
  float ms; (void)hipEventElapsedTime(&ms, a, b);
  double ops = 5.0 * blocks * 256.0 * kIters * 8.0;
  printf("%-6s %8.3f ms  %7.2f T lane-op/s\n", name, ms / 5, ops / (ms * 1e-3) / 1e12);
}
int main() {
  const int blocks = 256 * 8 * 4;  // 8192 workgroups of 256 lanes
  float* out; if (hipMalloc(&out, sizeof(float) * blocks * 256) != hipSuccess) return 1;
  run<0>("fma", out, blocks); run<1>("exp2", out, blocks); run<2>("rcp", out, blocks);
  run<3>("sqrt", out, blocks); run<4>("log2", out, blocks); run<0>("fma", out, blocks);
  run<5>("mul", out, blocks); run<6>("add", out, blocks); run<9>("dppmov", out, blocks); run<10>("fma3v", out, blocks);
  (void)hipFree(out);
  return hipDeviceSynchronize() == hipSuccess ? 0 : 1;
}
