// rope.hip -- rotary position embedding on gfx950: the (cos, sin) table and the standalone
// rotation of a [B, H, T, D] tensor.
//
// RoPE rotates adjacent pairs (x[2i], x[2i+1]) of a query or key row at position t by the angle
// t * theta^(-2i/D) (agentlenshq NanoEuler page, "기술 사양"; byte-level GPT page, "Core
// Mechanics": a rotation of queries and keys that encodes relative position).  The angle is
// formed and its cosine/sine evaluated in double, then rounded to float32: in float32 the angle
// t * w alone would carry an error of about t * 2^-24 rad (1e-4 rad at t = 2047).
#include "common.hpp"
#include "kernels.hpp"

namespace ne {

namespace {

__global__ __launch_bounds__(256) void rope_table_kernel(int rows, int D, double theta, float* cs) {
    const long n = (long)rows * (D / 2);
    const long gid = (long)blockIdx.x * 256 + threadIdx.x;
    if (gid >= n) return;
    const int t = (int)(gid / (D / 2));
    const int i = (int)(gid % (D / 2));
    const double w = pow(theta, -(2.0 * i) / (double)D);
    const double ang = (double)t * w;
    double s, c;
    sincos(ang, &s, &c);
    reinterpret_cast<f32x2*>(cs)[gid] = f32x2{(float)c, (float)s};
}

template <typename T, int D>
__global__ __launch_bounds__(256) void rope_apply_kernel(RopeArgs a) {
    constexpr int VEC = 16 / sizeof(T);
    const long n = (long)a.rows * (D / VEC);
    const long gid = (long)blockIdx.x * 256 + threadIdx.x;
    if (gid >= n) return;
    const long row = gid / (D / VEC);
    const int d0 = (int)(gid % (D / VEC)) * VEC;
    const int t = (int)(row % a.T) + a.pos_offset;
    float x[VEC];
    load16<T>(reinterpret_cast<const T*>(a.x) + row * D + d0, x);
    rope_rotate(x, VEC, a.rope_cs, D, t, d0, a.inverse != 0);
    store16<T>(reinterpret_cast<T*>(a.y) + row * D + d0, x);
}

}  // namespace

hipError_t launch_rope_table(int rows, int D, double theta, float* cs, hipStream_t stream) {
    const long n = (long)rows * (D / 2);
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, rows, D,
                       theta, cs);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_rope(const RopeArgs& a, hipStream_t stream) {
    constexpr int VEC = 16 / sizeof(T);
    const long n = (long)a.rows * (D / VEC);
    hipLaunchKernelGGL((rope_apply_kernel<T, D>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template hipError_t launch_rope<bf16, 128>(const RopeArgs&, hipStream_t);
template hipError_t launch_rope<float, 128>(const RopeArgs&, hipStream_t);
template hipError_t launch_rope<bf16, 64>(const RopeArgs&, hipStream_t);
template hipError_t launch_rope<bf16, 32>(const RopeArgs&, hipStream_t);
template hipError_t launch_rope<float, 64>(const RopeArgs&, hipStream_t);
template hipError_t launch_rope<float, 32>(const RopeArgs&, hipStream_t);

}  // namespace ne
