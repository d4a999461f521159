// K1: per-token preparation of new query/key/value rows.
//
// For each new token (b, s) at absolute position p = past_b + s:
//   * query heads (when requested): optional per-head RMSNorm with
//     q_norm_weight, optional rotary, written to a query workspace in BSH
//     order (GroupQueryAttention page, Inputs table: q/k_norm_weight are
//     applied before rotary; SparseAttention page, Inputs table: cos_cache
//     width fixes the rotated dims, Attributes table: rotary_interleaved);
//   * key heads: the same transform with k_norm_weight, then written to the
//     key cache row p;
//   * value heads: copied to the value cache row p.
// Cache rows other than p are never touched, so a shared or in-place cache
// keeps every unchanged row (GroupQueryAttention page, Implementation
// variants on retaining existing cache rows).
//
// One workgroup (4 waves) per token; each wave transforms one head at a
// time with its lanes spread over the head's dims.  The transformed head is
// staged in LDS so that a lane can read its rotary partner.
#include "device_common.hpp"
#include "kvattn_internal.hpp"

namespace kvattn {
namespace {

constexpr int kPrepThreads = 256;

template <typename T>
__global__ __launch_bounds__(kPrepThreads) void prep_kernel(PrepParams p) {
  __shared__ float row[4][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tok = blockIdx.x;
  const int b = tok / p.S, s = tok % p.S;
  const int H = p.H;

  int past = 0;
  if (p.pos_mode == 1) past = p.lens[b] + 1 - p.S;
  else if (p.pos_mode == 2) past = p.lens[b] - p.S;
  const int pos = past + s;

  const int nq = p.write_q ? p.N : 0;
  const int nk = p.write_kv ? p.kvN : 0;
  const int total = nq + 2 * nk;
  const T* cs = static_cast<const T*>(p.cos);
  const T* sn = static_cast<const T*>(p.sin);
  const int rpos = (cs != nullptr) ? min(max(pos, 0), p.rot_rows - 1) : 0;
  const bool row_ok = pos >= 0 && pos < p.cap;

  for (int base = 0; base < total; base += 4) {
    const int item = base + wave;
    if (item < total) {
      int kind, h;  // kind 0 = query, 1 = key, 2 = value
      if (item < nq) { kind = 0; h = item; }
      else if (item < nq + nk) { kind = 1; h = item - nq; }
      else { kind = 2; h = item - nq - nk; }
      const T* src;
      if (kind == 0) src = static_cast<const T*>(p.q) + (int64_t)tok * p.q_stride + p.q_off + (int64_t)h * H;
      else if (kind == 1) src = static_cast<const T*>(p.k) + (int64_t)tok * p.k_stride + p.k_off + (int64_t)h * H;
      else src = static_cast<const T*>(p.v) + (int64_t)tok * p.v_stride + p.v_off + (int64_t)h * H;

      if (kind == 2) {
        if (row_ok) {
          T* dst = static_cast<T*>(p.vc) + (((int64_t)b * p.kvN + h) * p.cap + pos) * H;
          for (int d = lane; d < H; d += 64) dst[d] = src[d];
        }
      } else {
        const T* nw = static_cast<const T*>(kind == 0 ? p.q_norm : p.k_norm);
        float x[4];
        float ss = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          int d = lane + 64 * u;
          x[u] = (d < H) ? to_f32(src[d]) : 0.f;
          ss += x[u] * x[u];
        }
        if (nw != nullptr) {
          ss = wave_sum_xor(ss, 1, 32);
          float r = rsqrtf(ss / (float)H + p.eps);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            int d = lane + 64 * u;
            if (d < H) x[u] *= r * to_f32(nw[d]);
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) row[wave][lane + 64 * u] = x[u];
        // the row is private to this wave: a wave-scope fence orders the
        // lanes' LDS writes before the partner reads below
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float y[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          int d = lane + 64 * u;
          y[u] = x[u];
          if (cs != nullptr && d < 2 * p.rot_half) {
            int i, partner;
            float sign;
            if (p.interleaved) {
              i = d >> 1;
              partner = d ^ 1;
              sign = (d & 1) ? 1.f : -1.f;
            } else {
              i = d < p.rot_half ? d : d - p.rot_half;
              partner = d < p.rot_half ? d + p.rot_half : d - p.rot_half;
              sign = d < p.rot_half ? -1.f : 1.f;
            }
            float co = to_f32(cs[(int64_t)rpos * p.rot_half + i]);
            float si = to_f32(sn[(int64_t)rpos * p.rot_half + i]);
            // first of a pair: a*cos - b*sin; second: b*cos + a*sin
            y[u] = x[u] * co + sign * row[wave][partner] * si;
          }
        }
        if (kind == 0) {
          T* dst = static_cast<T*>(p.q_out) + ((int64_t)tok * p.N + h) * H;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            int d = lane + 64 * u;
            if (d < H) dst[d] = from_f32<T>(y[u]);
          }
        } else if (row_ok) {
          T* dst = static_cast<T*>(p.kc) + (((int64_t)b * p.kvN + h) * p.cap + pos) * H;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            int d = lane + 64 * u;
            if (d < H) dst[d] = from_f32<T>(y[u]);
          }
        }
      }
    }
    __syncthreads();
  }
}

template <typename T>
__global__ __launch_bounds__(256) void copy_past_kernel(CopyPastParams p) {
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int total = p.lens[b] + 1;
  int rows = total - p.S;
  rows = min(rows, min(p.past_seq, p.cap));
  if (rows <= 0) return;
  const int64_t n = (int64_t)rows * p.H;
  const T* sk = static_cast<const T*>(p.pk) + ((int64_t)b * p.kvN + kvh) * p.past_seq * p.H;
  const T* sv = static_cast<const T*>(p.pv) + ((int64_t)b * p.kvN + kvh) * p.past_seq * p.H;
  T* dk = static_cast<T*>(p.ck) + ((int64_t)b * p.kvN + kvh) * p.cap * p.H;
  T* dv = static_cast<T*>(p.cv) + ((int64_t)b * p.kvN + kvh) * p.cap * p.H;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    dk[i] = sk[i];
    dv[i] = sv[i];
  }
}

}  // namespace

hipError_t launch_prep(DType dt, const PrepParams& p, hipStream_t s) {
  if (p.B * p.S == 0) return hipSuccess;
  dim3 grid(p.B * p.S);
  if (dt == DType::F16)
    hipLaunchKernelGGL(prep_kernel<f16>, grid, dim3(kPrepThreads), 0, s, p);
  else
    hipLaunchKernelGGL(prep_kernel<float>, grid, dim3(kPrepThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_copy_past(DType dt, const CopyPastParams& p, hipStream_t s) {
  int64_t per = (int64_t)p.past_seq * p.H;
  int gx = (int)std::min<int64_t>((per + 255) / 256, 1024);
  if (gx < 1) gx = 1;
  dim3 grid(gx, p.kvN, p.B);
  if (dt == DType::F16)
    hipLaunchKernelGGL(copy_past_kernel<f16>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(copy_past_kernel<float>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvattn
