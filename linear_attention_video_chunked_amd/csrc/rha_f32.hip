// float32 path: the same hybrid attention and chunk states with all arithmetic
// in IEEE float32 (vector ALU, no matrix cores).  Used for RHA_F32 problems,
// where the result must track a float64 reference to ~1e-5.
//
// Forward: one thread per query row, 128 rows per workgroup; K/V tiles of 32
// keys are staged in LDS and read by broadcast.  The linear term
// phi(q)^T S_c, phi(q).z_c seeds the numerator and denominator at reference
// maximum 0 ("Long-Horizon Streaming Video Generation via Hybrid Attention with
// Decoupled Distillation", explainer section 2.A, with the shared normaliser);
// the online maximum then follows every key.
// Chunk state: one workgroup per (head, chunk), each thread an 8x8 block of
// U = phi(K)^T V, tokens staged through LDS in tiles of 32.
#include "rha_device.hpp"
#include "rha_launch.hpp"

namespace rha {
namespace {

constexpr int FBM = 128;  // query rows per workgroup
constexpr int FBN = 32;   // keys per tile

__device__ __forceinline__ float phi_f32(float x) { return x > 0.f ? x + 1.f : expf(x); }

template <int D>
__global__ __launch_bounds__(FBM) void fwd_f32_kernel(const FwdParams p) {
  __shared__ __attribute__((aligned(16))) float ks[FBN][D];
  __shared__ __attribute__((aligned(16))) float vs[FBN][D];
  const int tid = threadIdx.x;

  const int tile = blockIdx.x % p.tiles_per_chunk;
  const int rest = blockIdx.x / p.tiles_per_chunk;
  const int c = rest % p.n_qchunks;
  const int bh = rest / p.n_qchunks;
  const int b = bh / p.H, h = bh % p.H;
  const int qrow0 = tile * FBM;
  const int nrows = min(FBM, p.C - qrow0);
  const int64_t qtok0 = (int64_t)c * p.C + qrow0;
  const bool ok = tid < nrows;

  const float* qrow = (const float*)p.q + b * p.q_sb + h * p.q_sh + (qtok0 + tid) * p.q_st;
  const float* kbase = (const float*)p.k + b * p.kv_sb + h * p.kv_sh;
  const float* vbase = (const float*)p.v + b * p.kv_sb + h * p.kv_sh;

  int64_t kbeg, kend;
  bool has_state;
  const float* Sp;
  const float* zp;
  if (!p.stream_mode) {
    if (p.w > 0) {
      kbeg = (int64_t)max(0, c - p.w + 1) * p.C;
      kend = (int64_t)(c + 1) * p.C;
    } else {
      kbeg = kend = 0;
    }
    has_state = (p.w == 0) || (c >= p.w);
    Sp = p.S + ((int64_t)bh * p.n_qchunks + c) * D * D;
    zp = p.z + ((int64_t)bh * p.n_qchunks + c) * D;
  } else {
    kbeg = 0;
    kend = p.n_keys;
    has_state = p.has_state != 0;
    Sp = p.S + (int64_t)bh * D * D;
    zp = p.z + (int64_t)bh * D;
  }

  float q[D], acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = ok ? qrow[e] : 0.f;
    acc[e] = 0.f;
  }
  float m, l = 0.f;
  if (has_state) {
    // S staged 32 rows at a time through the K buffer
    for (int e0 = 0; e0 < D; e0 += FBN) {
      for (int i = tid; i < FBN * D; i += FBM) ks[i / D][i % D] = Sp[(int64_t)(e0 + i / D) * D + i % D];
      __syncthreads();
#pragma unroll
      for (int e = 0; e < FBN; ++e) {
        const float f = phi_f32(q[e0 + e]);
#pragma unroll
        for (int n = 0; n < D; ++n) acc[n] = fmaf(f, ks[e][n], acc[n]);
      }
      __syncthreads();
    }
#pragma unroll
    for (int e = 0; e < D; ++e) l = fmaf(phi_f32(q[e]), zp[e], l);
    m = 0.f;
  } else {
    m = -INFINITY;
  }

  const float scale = rsqrtf((float)D);
  for (int64_t k0 = kbeg; k0 < kend; k0 += FBN) {
    const int valid = (int)min((int64_t)FBN, kend - k0);
    for (int i = tid; i < FBN * D; i += FBM) {
      const int r = i / D, e = i % D;
      const bool in = r < valid;
      ks[r][e] = in ? kbase[(k0 + r) * p.kv_st + e] : 0.f;
      vs[r][e] = in ? vbase[(k0 + r) * p.kv_st + e] : 0.f;
    }
    __syncthreads();
    for (int j = 0; j < valid; ++j) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) s = fmaf(q[e], ks[j][e], s);
      s *= scale;
      if (s > m) {
        const float alpha = expf(m - s);
        l *= alpha;
#pragma unroll
        for (int n = 0; n < D; ++n) acc[n] *= alpha;
        m = s;
      }
      const float pj = expf(s - m);
      l += pj;
#pragma unroll
      for (int n = 0; n < D; ++n) acc[n] = fmaf(pj, vs[j][n], acc[n]);
    }
    __syncthreads();
  }

  if (ok) {
    float* orow = (float*)p.out + b * p.q_sb + h * p.q_sh + (qtok0 + tid) * p.q_st;
    const float inv = 1.0f / l;
#pragma unroll
    for (int n = 0; n < D; ++n) orow[n] = acc[n] * inv;
    if (p.lse != nullptr) {
      const int64_t L = (int64_t)p.n_qchunks * p.C;
      p.lse[(int64_t)bh * L + qtok0 + tid] = m + logf(l);
    }
  }
}

constexpr int FST = 256;  // threads of the chunk-state kernel
constexpr int FBT = 32;   // tokens per tile

template <int D>
__global__ __launch_bounds__(FST) void chunk_state_f32_kernel(const ChunkStateParams p) {
  __shared__ __attribute__((aligned(16))) float fk[FBT][D];
  __shared__ __attribute__((aligned(16))) float vv[FBT][D];
  const int tid = threadIdx.x;
  const int jc = blockIdx.x % p.n_chunks;
  const int bh = blockIdx.x / p.n_chunks;
  const int b = bh / p.H, h = bh % p.H;
  const int64_t t0 = (int64_t)(p.chunk0 + jc) * p.C;
  const int len = (int)min((int64_t)p.C, p.tok_end - t0);  // tokens of this chunk
  const float* kbase = (const float*)p.k + b * p.kv_sb + h * p.kv_sh + t0 * p.kv_st;
  const float* vbase = (const float*)p.v + b * p.kv_sb + h * p.kv_sh + t0 * p.kv_st;

  constexpr int NBLK = D / 8;
  const bool active = tid < NBLK * NBLK;
  const int e0 = (tid / NBLK) * 8, n0 = (tid % NBLK) * 8;
  float acc[8][8], zs[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    zs[i] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
  }

  for (int tb = 0; tb < len; tb += FBT) {
    const int valid = min(FBT, len - tb);
    for (int i = tid; i < FBT * D; i += FST) {
      const int r = i / D, e = i % D;
      const bool in = r < valid;
      fk[r][e] = in ? phi_f32(kbase[(int64_t)(tb + r) * p.kv_st + e]) : 0.f;
      vv[r][e] = in ? vbase[(int64_t)(tb + r) * p.kv_st + e] : 0.f;
    }
    __syncthreads();
    if (active) {
      for (int t = 0; t < valid; ++t) {
        float a[8], bv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          a[i] = fk[t][e0 + i];
          bv[i] = vv[t][n0 + i];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          zs[i] += a[i];
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], bv[j], acc[i][j]);
        }
      }
    }
    __syncthreads();
  }

  if (active) {
    float* Sdst = p.S + (int64_t)bh * p.s_bh + (int64_t)(jc + p.slot_offset) * D * D;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float* dst = Sdst + (int64_t)(e0 + i) * D + n0 + j;
        *dst = p.accumulate ? *dst + acc[i][j] : acc[i][j];
      }
    if (n0 == 0) {
      float* zd = p.z + (int64_t)bh * p.z_bh + (int64_t)(jc + p.slot_offset) * D + e0;
#pragma unroll
      for (int i = 0; i < 8; ++i) zd[i] = p.accumulate ? zd[i] + zs[i] : zs[i];
    }
  }
}

}  // namespace

hipError_t launch_fwd_f32(FwdParams& p, int d, hipStream_t s) {
  p.tiles_per_chunk = (p.C + FBM - 1) / FBM;
  p.total_tiles = p.B * p.H * p.n_qchunks * p.tiles_per_chunk;
  if (p.total_tiles == 0) return hipSuccess;
  if (d == 128)
    hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3(p.total_tiles), dim3(FBM), 0, s, p);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3(p.total_tiles), dim3(FBM), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_chunk_state_f32(const ChunkStateParams& p, int d, hipStream_t s) {
  const dim3 grid((unsigned)(p.B * p.H * p.n_chunks));
  if (d == 128)
    hipLaunchKernelGGL(chunk_state_f32_kernel<128>, grid, dim3(FST), 0, s, p);
  else
    hipLaunchKernelGGL(chunk_state_f32_kernel<64>, grid, dim3(FST), 0, s, p);
  return hipGetLastError();
}

}  // namespace rha
