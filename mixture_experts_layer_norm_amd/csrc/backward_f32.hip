// fp32 backward of the expert FFN (the fp32 path serves small configurations; the BF16 and MXFP8
// paths carry the large ones). Same steps as the BF16 backward (sparsenotes page "Mixture-of-Kittens:
// MoE Megakernel for NVL72s": replay of a and u instead of stored activations, "A ring buffer instead
// of a host round-trip"; the router-weight gradient dg = <h, W_down^T dy>, "The production details"),
// every operand in fp32, so no operand splitting is needed:
//   replay     a = x W_gate^T, u = x W_up^T
//   dgrad-down dh' = dy W_down;  dg = <h, dh'>;  dh = g dh'
//   SwiGLU     da = dh u sig(a) (1 + a (1 - sig(a))),  du = dh SiLU(a)
//   dgrad-up   dx = da W_gate + du W_up
//   wgrad      dW_down = sum_j g_j dy_j h_j^T,  dW_gate = sum_j da_j x_j^T,  dW_up = sum_j du_j x_j^T
// One strided GEMM kernel reads every operand in place (no transposes): A(m, k) = A[m sam + k sak],
// B(k, n) = B[k sbk + n sbn]; each output element is summed by one thread with k ascending.
#include "common.h"

namespace moe {

struct F32Gemm {
  const float* A = nullptr; int64_t sam = 0, sak = 0;
  const float* B = nullptr; int64_t sbk = 0, sbn = 0, b_group_stride = 0;
  float* C = nullptr; int64_t ldc = 0, c_group_stride = 0;
  const float* kscale = nullptr;   // A(m, k) * kscale[k] (k a slot row; weight-gradient GEMMs)
  int M = 0, N = 0, K = 0;
  int accumulate = 0;              // C += product instead of C = product
};

// Row-grouped (KG = false): group g = blockIdx.z owns rows offs[g] .. offs[g+1]-1 of A and C and
// the weights B + g * b_group_stride; m-tile blockIdx.y of 64 rows inside the group, K = a.K.
// K-grouped (KG = true): group g contracts k over offs[g] .. offs[g+1]-1 (slot rows) into
// C + g * c_group_stride [M][ldc]; an empty group writes zeros.
// 64 x 64 tile, 256 threads of 4 x 4 outputs, K staged through LDS 16 at a time.
template <bool KG>
__global__ __launch_bounds__(256) void gemm_f32s_kernel(F32Gemm a, const int32_t* __restrict__ offs) {
  __shared__ float As[16][64 + 1];
  __shared__ float Bs[16][64 + 1];
  const int g = blockIdx.z, tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int n0 = blockIdx.x * 64;
  int m0, mend, k_lo, k_hi;
  if (KG) {
    m0 = blockIdx.y * 64;
    mend = a.M;
    k_lo = offs[g];
    k_hi = offs[g + 1];
  } else {
    m0 = offs[g] + blockIdx.y * 64;
    mend = offs[g + 1];
    if (m0 >= mend) return;
    k_lo = 0;
    k_hi = a.K;
  }
  const float* B = a.B + (KG ? 0 : (int64_t)g * a.b_group_stride);
  float acc[4][4] = {};
  for (int k0 = k_lo; k0 < k_hi; k0 += 16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q, kk = e >> 6, mm = e & 63;
      const int k = k0 + kk, m = m0 + mm;
      float v = 0.f;
      if (k < k_hi && m < mend) {
        v = a.A[(int64_t)m * a.sam + (int64_t)k * a.sak];
        if (a.kscale) v *= a.kscale[k];
      }
      As[kk][mm] = v;
      const int n = n0 + mm;
      Bs[kk][mm] = (k < k_hi && n < a.N) ? B[(int64_t)k * a.sbk + (int64_t)n * a.sbn] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(As[kk][ty * 4 + i], Bs[kk][tx * 4 + j], acc[i][j]);
    __syncthreads();
  }
  float* C = a.C + (KG ? (int64_t)g * a.c_group_stride : 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= mend) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= a.N) continue;
      float* c = C + (int64_t)m * a.ldc + n;
      *c = a.accumulate ? *c + acc[i][j] : acc[i][j];
    }
  }
}

// grid: row-grouped (ceil(N / 64), ceil(max rows of a group / 64), G); K-grouped (ceil(N / 64),
// ceil(M / 64), G). max_rows bounds every group's rows (row-grouped) on the host.
static int launch_gemm_f32s(const F32Gemm& a, bool kg, const int32_t* offs, int G, int64_t max_rows, hipStream_t s) {
  if (G <= 0 || a.N <= 0) return MOE_OK;
  const int64_t gy = kg ? (a.M + 63) / 64 : (max_rows + 63) / 64;
  if (gy <= 0) return MOE_OK;
  if (gy > 65535 || G > 65535) return MOE_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)((a.N + 63) / 64), (unsigned)gy, (unsigned)G);
  if (kg)
    hipLaunchKernelGGL(gemm_f32s_kernel<true>, grid, dim3(256), 0, s, a, offs);
  else
    hipLaunchKernelGGL(gemm_f32s_kernel<false>, grid, dim3(256), 0, s, a, offs);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

// One wavefront per slot row j < n: from a, u, dh' (fp32 [n][I]) and the row weight g (nullable:
// 1), h -> hf, da -> daf, du -> duf, and dg[j] = sum_i h_i dh'_i (nullable; per-lane sums in unit
// order, then a fixed butterfly).
__global__ __launch_bounds__(256) void swiglu_bwd_f32_kernel(const float* __restrict__ a, const float* __restrict__ u,
                                                             const float* __restrict__ dhp, const float* __restrict__ g,
                                                             int64_t n, int I, float* __restrict__ hf,
                                                             float* __restrict__ daf, float* __restrict__ duf,
                                                             float* __restrict__ dg) {
  const int lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= n) return;
  const float gj = g ? g[j] : 1.f;
  float part = 0.f;
  for (int i = lane; i < I; i += 64) {
    const int64_t e = j * I + i;
    const float x = a[e], uu = u[e], p = dhp[e];
    const float sg = sigmoid_f(x), sa = x * sg, h = sa * uu, dh = gj * p;
    hf[e] = h;
    daf[e] = dh * uu * sg * (1.f + x * (1.f - sg));
    duf[e] = dh * sa;
    part = fmaf(h, p, part);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
  if (dg && lane == 0) dg[j] = part;
}

// dx[t] = dx_shared[t] (nullable: 0) + sum_k dx_slot[inv_perm[t K + k]], k ascending.
__global__ __launch_bounds__(256) void reverse_dispatch_f32_kernel(const float* __restrict__ dxs,
                                                                   const int32_t* __restrict__ inv_perm,
                                                                   const float* __restrict__ dsh, float* __restrict__ dx,
                                                                   int T, int K, int D) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)T * D) return;
  const int64_t t = i / D, d = i % D;
  float acc = dsh ? dsh[i] : 0.f;
  for (int k = 0; k < K; ++k) acc += dxs[(int64_t)inv_perm[t * K + k] * D + d];
  dx[i] = acc;
}

int launch_reverse_dispatch_f32(const float* dx_slot, const int32_t* inv_perm, const float* dx_shared, float* dx, int T,
                                int K, int D, hipStream_t s) {
  const int64_t n = (int64_t)T * D;
  if (n == 0) return MOE_OK;
  hipLaunchKernelGGL(reverse_dispatch_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dx_slot, inv_perm,
                     dx_shared, dx, T, K, D);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

// Backward of G groups of rows (offs: sanitised offsets, rows offs[g] .. offs[g+1]-1 of x_rows,
// dy_rows [n][D] fp32) through W_gate, W_up [G][I][D] and W_down [G][D][I] (fp32). g_rows
// nullable (weight 1: the shared expert); dg_rows nullable. Scratch: a, u, dh', h, da, du [n][I].
int core_backward_f32(int G, int64_t n_cap, int64_t max_rows, int D, int I, const float* x_rows, const float* dy_rows,
                      const float* g_rows, const int32_t* offs, const float* wg, const float* wu, const float* wd,
                      float* dx_rows, float* dg_rows, float* dw_gate, float* dw_up, float* dw_down, float* sa, float* su,
                      float* sdh, float* sh, float* sda, float* sdu, hipStream_t s) {
  int st;
  const int64_t ID = (int64_t)I * D;
  F32Gemm r;   // replay: a = x W_gate^T (then u with W_up)
  r.A = x_rows; r.sam = D; r.sak = 1; r.B = wg; r.sbk = 1; r.sbn = D; r.b_group_stride = ID;
  r.C = sa; r.ldc = I; r.N = I; r.K = D;
  if ((st = launch_gemm_f32s(r, false, offs, G, max_rows, s))) return st;
  r.B = wu; r.C = su;
  if ((st = launch_gemm_f32s(r, false, offs, G, max_rows, s))) return st;
  F32Gemm d;   // dgrad-down: dh' = dy W_down
  d.A = dy_rows; d.sam = D; d.sak = 1; d.B = wd; d.sbk = I; d.sbn = 1; d.b_group_stride = ID;
  d.C = sdh; d.ldc = I; d.N = I; d.K = D;
  if ((st = launch_gemm_f32s(d, false, offs, G, max_rows, s))) return st;
  if (n_cap > 0) {
    hipLaunchKernelGGL(swiglu_bwd_f32_kernel, dim3((unsigned)((n_cap + 3) / 4)), dim3(256), 0, s, sa, su, sdh, g_rows,
                       n_cap, I, sh, sda, sdu, dg_rows);
    MOE_LAUNCH_CHECK();
  }
  F32Gemm u;   // dgrad-up: dx = da W_gate + du W_up
  u.A = sda; u.sam = I; u.sak = 1; u.B = wg; u.sbk = D; u.sbn = 1; u.b_group_stride = ID;
  u.C = dx_rows; u.ldc = D; u.N = D; u.K = I;
  if ((st = launch_gemm_f32s(u, false, offs, G, max_rows, s))) return st;
  u.A = sdu; u.B = wu; u.accumulate = 1;
  if ((st = launch_gemm_f32s(u, false, offs, G, max_rows, s))) return st;
  F32Gemm w;   // dW_down[g] = sum_j g_j dy_j h_j^T  ([D][I])
  w.A = dy_rows; w.sam = 1; w.sak = D; w.kscale = g_rows; w.B = sh; w.sbk = I; w.sbn = 1;
  w.C = dw_down; w.ldc = I; w.c_group_stride = ID; w.M = D; w.N = I;
  if ((st = launch_gemm_f32s(w, true, offs, G, 0, s))) return st;
  F32Gemm v;   // dW_gate[g] = sum_j da_j x_j^T, dW_up[g] = sum_j du_j x_j^T  ([I][D])
  v.A = sda; v.sam = 1; v.sak = I; v.B = x_rows; v.sbk = D; v.sbn = 1;
  v.C = dw_gate; v.ldc = D; v.c_group_stride = ID; v.M = I; v.N = D;
  if ((st = launch_gemm_f32s(v, true, offs, G, 0, s))) return st;
  v.A = sdu; v.C = dw_up;
  return launch_gemm_f32s(v, true, offs, G, 0, s);
}

}  // namespace moe
