// C ABI of libmla.so: host-side validation, workspace carving and dispatch.
// See include/mla.h for the contract of every entry point.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <mutex>
#include <vector>

#include "mla.h"
#include "mla_internal.hpp"

namespace {

thread_local char g_err[512] = "";

// Events for the next attention call on this thread (mla_time_next_attn).
struct AttnTiming {
  hipEvent_t start = nullptr, kernel_end = nullptr, call_end = nullptr;
};
thread_local AttnTiming g_attn_timing;

AttnTiming take_attn_timing() {
  const AttnTiming t = g_attn_timing;
  g_attn_timing = AttnTiming{};
  return t;
}

mla_status fail(mla_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

mla_status ok() {
  g_err[0] = '\0';
  return MLA_OK;
}

size_t elem_size(int dtype) { return dtype == MLA_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

mla_status check_dims(const mla_dims* d) {
  if (!d) return fail(MLA_ERR_NULL, "dims is NULL");
  if (d->dtype != MLA_FP32 && d->dtype != MLA_BF16) return fail(MLA_ERR_DTYPE, "dtype %d", d->dtype);
  if (d->d <= 0 || d->H <= 0 || d->d_h <= 0 || d->d_v <= 0 || d->d_c <= 0 || d->d_R <= 0 || d->d_cq < 0)
    return fail(MLA_ERR_SHAPE, "non-positive size in dims");
  if (d->d_R % 2) return fail(MLA_ERR_SHAPE, "d_R must be even (rotary pairs)");
  if (d->d_c > 1024 || d->d_c + d->d_R > 2048)
    return fail(MLA_ERR_UNSUPPORTED, "d_c > 1024 or d_c + d_R > 2048");
  if (!(d->rope_theta > 0.f)) return fail(MLA_ERR_SHAPE, "rope_theta must be > 0");
  if (d->softmax_scale < 0.f || std::isnan(d->softmax_scale)) return fail(MLA_ERR_SHAPE, "softmax_scale");
  // Rows must be 16-byte multiples so every row start stays 16-byte aligned.
  if (((d->d_c + d->d_R) * elem_size(d->dtype)) % 16)
    return fail(MLA_ERR_ALIGN, "cache row bytes must be a multiple of 16");
  return MLA_OK;
}

float softmax_scale(const mla_dims* d) {
  return d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / std::sqrt(static_cast<float>(d->d_h + d->d_R));
}

mla_status check_cache(const mla_dims* d, const mla_cache* c) {
  if (!c) return fail(MLA_ERR_NULL, "cache is NULL");
  if (!c->data) return fail(MLA_ERR_NULL, "cache.data is NULL");
  if (!aligned16(c->data)) return fail(MLA_ERR_ALIGN, "cache.data not 16-byte aligned");
  if (c->block_table) {
    if (c->block_size <= 0 || c->max_blocks <= 0 || c->n_blocks <= 0)
      return fail(MLA_ERR_SHAPE, "paged cache sizes must be positive");
    if (c->block_size & (c->block_size - 1)) return fail(MLA_ERR_UNSUPPORTED, "block_size must be a power of two");
    if (!aligned16(c->block_table)) return fail(MLA_ERR_ALIGN, "block_table not 16-byte aligned");
  } else if (c->capacity <= 0) {
    return fail(MLA_ERR_SHAPE, "contiguous cache capacity must be positive");
  }
  (void)d;
  return MLA_OK;
}

int device_cus() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return 256;
  return v;
}

bool mfma_attn(const mla_dims* d) {
  return d->dtype == MLA_BF16 && d->d_c == 512 && d->d_R == 64 && d->H % 32 == 0 && d->H <= 128;
}

// MFMA attention: workgroups launched. Explicit splits: num_splits per
// sequence (at most); balanced plan: one per compute unit, at least one per
// sequence. The device cuts the sequences into chunks that fit this grid.
constexpr int kMaxMfmaBatch = 32768;   // plan scratch: B ints of LDS
constexpr int kMinChunk = 128;         // rows; the device plan's lower bound on the chunk size
int cdiv(long long a, long long b) { return static_cast<int>((a + b - 1) / b); }
// explicit split count, clamped to the tiles of the longest sequence (more
// would give the same chunks); 0 = balanced plan
int mfma_splits(int num_splits, int max_seq_len) {
  return num_splits > 0 ? std::min(num_splits, std::max(1, cdiv(max_seq_len, 32))) : 0;
}
long long mfma_grid(int B, int splits) {
  return splits > 0 ? static_cast<long long>(B) * splits : std::max(device_cus(), B);
}
constexpr long long kMaxMfmaGrid = 1LL << 22;
// Chunks the device plan gives a sequence of length L when all B sequences
// have that length (the plan itself runs on the device from seq_lens).
int mfma_uniform_chunks(int B, int L, int num_splits, int grid) {
  auto chunks = [&](int t) {
    const int c = std::max(32, cdiv(cdiv(L, t), 32) * 32);
    return std::max(1, cdiv(L, c));
  };
  if (num_splits > 0) return chunks(num_splits);
  int klo = cdiv(std::max(kMinChunk, cdiv(std::max(static_cast<long long>(B) * L, 1LL), grid)), 32);
  int khi = std::max(klo, cdiv(std::max(L, 1), 32));
  while (klo < khi) {
    const int mid = (klo + khi) / 2;
    if (static_cast<long long>(B) * std::max(1, cdiv(L, mid * 32)) <= grid) khi = mid;
    else klo = mid + 1;
  }
  return chunks(std::max(1, cdiv(L, klo * 32)));
}

// Split count and rows per split for the generic attention launch.
void attn_plan(const mla_dims* d, int B, int max_seq_len, int num_splits, int* splits, int* chunk) {
  const int L = max_seq_len > 0 ? max_seq_len : 1;
  int s = num_splits;
  if (s <= 0) {
    const int cus = device_cus();
    s = (cus + B - 1) / B;                  // about one workgroup per compute unit
    const int min_rows = 256;
    const int smax = (L + min_rows - 1) / min_rows;
    if (s > smax) s = smax;
    if (s < 1) s = 1;
  }
  if (s > L) s = L;
  int ch = (L + s - 1) / s;
  if (mfma_attn(d)) ch = (ch + 31) / 32 * 32;   // whole 32-row tiles per split
  *chunk = ch;
  *splits = (L + ch - 1) / ch;
}

struct GemmShape { int M, N, K, G; };

int splits_for(const GemmShape& s, int dtype) { return mla::gemm_splits(s.M, s.N, s.K, s.G, dtype); }

size_t part_bytes(const GemmShape& s, int dtype) {
  return static_cast<size_t>(splits_for(s, dtype)) * s.G * s.M * s.N * sizeof(float);
}

size_t ws_compress(const mla_dims* d, int B) {
  // two products' partials, or one concatenated product's
  return std::max(align_up(part_bytes({B, d->d_c, d->d, 1}, d->dtype)) + align_up(part_bytes({B, d->d_R, d->d, 1}, d->dtype)),
                  align_up(part_bytes({B, d->d_c + d->d_R, d->d, 1}, d->dtype)));
}

// The query side keeps its intermediates c_Q and q_C in float32, so that the
// products feeding the scores (W_QR, W_UK^T) can read them as two bf16 terms;
// c_Q also in bf16 (bf16 storage), for W_UQ, which takes it rounded once.
size_t ws_absorb(const mla_dims* d, int B) {
  const size_t es = sizeof(float);
  const int qin = d->d_cq ? d->d_cq : d->d;
  size_t p = 0;
  if (d->d_cq) p = part_bytes({B, d->d_cq, d->d, 1}, d->dtype);
  p = std::max(p, part_bytes({B, d->H * d->d_h, qin, 1}, d->dtype));
  p = std::max(p, part_bytes({B, d->H * d->d_R, qin, 1}, d->dtype));
  p = std::max(p, part_bytes({B, d->d_c, d->d_h, d->H}, d->dtype));
  return align_up(static_cast<size_t>(B) * d->d_cq * es) + align_up(static_cast<size_t>(B) * d->d_cq * 2) +
         align_up(static_cast<size_t>(B) * d->H * d->d_h * es) + align_up(p);
}

// MFMA path: partial O (fp16, scaled) and (m, l, E) per chunk of the grid,
// then the plan's per-sequence (first chunk, chunks).
size_t ws_attn_mfma(const mla_dims* d, int B, int max_seq_len, int num_splits) {
  const size_t g = static_cast<size_t>(std::min(kMaxMfmaGrid, mfma_grid(B, mfma_splits(num_splits, max_seq_len))));
  return align_up(g * d->H * d->d_c * 2) + align_up(g * d->H * 4 * sizeof(float)) +
         align_up(static_cast<size_t>(B) * 2 * sizeof(int));
}
size_t ws_attn(const mla_dims* d, int B, int max_seq_len, int num_splits) {
  if (mfma_attn(d)) return ws_attn_mfma(d, B, max_seq_len, num_splits);
  int s = 1, ch = 1;
  attn_plan(d, B, max_seq_len, num_splits, &s, &ch);
  if (s <= 1) return 0;
  return align_up(static_cast<size_t>(B) * s * d->H * d->d_c * sizeof(float)) +
         align_up(static_cast<size_t>(B) * s * d->H * 2 * sizeof(float));
}

// precomposed variant: c_Q, then partials of W_DQ, of the per-head W_QK
// product and of W_QR; the output product over H*d_c inputs
size_t ws_absorb_pre(const mla_dims* d, int B) {
  const size_t es = sizeof(float);   // c_Q in float32, as in ws_absorb
  const int qin = d->d_cq ? d->d_cq : d->d;
  size_t p = 0;
  if (d->d_cq) p = part_bytes({B, d->d_cq, d->d, 1}, d->dtype);
  p = std::max(p, part_bytes({B, d->d_c, qin, d->H}, d->dtype));
  p = std::max(p, part_bytes({B, d->H * d->d_R, qin, 1}, d->dtype));
  return align_up(static_cast<size_t>(B) * d->d_cq * es) + align_up(static_cast<size_t>(B) * d->d_cq * 2) +
         align_up(p);
}
size_t ws_out_pre(const mla_dims* d, int B) { return align_up(part_bytes({B, d->d, d->H * d->d_c, 1}, d->dtype)); }

size_t ws_out(const mla_dims* d, int B) {
  return align_up(std::max(part_bytes({B, d->d_v, d->d_c, d->H}, d->dtype),
                           part_bytes({B, d->d, d->H * d->d_v, 1}, d->dtype)));
}

mla_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MLA_OK;
}

#define MLA_TRY(expr)               \
  do {                              \
    mla_status _s = (expr);         \
    if (_s != MLA_OK) return _s;    \
  } while (0)

// a_split: a float32 activation enters as two bf16 terms (about float32
// precision for twice the MFMAs) instead of being rounded once to bf16.
mla_status gemm(const void* A, long long lda, long long sAg, bool a_f32, const void* W, long long ldw,
                long long sWg, bool w_kn, const GemmShape& s, int dtype, float* P, hipStream_t st,
                bool a_split = false) {
  mla::GemmArgs g{A, lda, sAg, a_f32, W, ldw, sWg, w_kn, s.M, s.N, s.K, s.G, splits_for(s, dtype), P, dtype};
  g.a_split = a_split;
  return hip_status(mla::launch_gemm(g, st), "gemm launch");
}

// Product stored to out[g*sOg + m*ldo + n] in dtype: directly by the GEMM when
// it runs as one split, else through fp32 partials P and the reduce epilogue.
// out_dtype: element type of out (MLA_FP32 or MLA_BF16); -1 = the storage dtype.
mla_status gemm_store(const void* A, long long lda, long long sAg, bool a_f32, const void* W, long long ldw,
                      long long sWg, bool w_kn, const GemmShape& s, int dtype, float* P, void* out,
                      long long ldo, long long sOg, hipStream_t st, int out_dtype = -1, bool a_split = false) {
  if (out_dtype < 0) out_dtype = dtype;
  mla::GemmArgs g{A, lda, sAg, a_f32, W, ldw, sWg, w_kn, s.M, s.N, s.K, s.G, splits_for(s, dtype), P, dtype};
  g.a_split = a_split;
  g.out = out;
  g.ldo = ldo;
  g.sOg = sOg;
  g.out_dtype = out_dtype;
  if (mla::gemm_direct(g)) return hip_status(mla::launch_gemm(g, st), "gemm launch");
  g.out = nullptr;
  MLA_TRY(hip_status(mla::launch_gemm(g, st), "gemm launch"));
  return hip_status(mla::launch_reduce_store(P, g.splits, s.G, s.M, s.N, out, ldo, sOg, out_dtype, st),
                    "reduce launch");
}

// c_Q = W_DQ h in float32 and, with bf16 storage, a bf16 copy (the split
// partials summed once into both).
mla_status cq_product(const void* h_t, bool f32, const void* W_DQ, const GemmShape& s, int dt, float* P, void* cq,
                      void* cq16, hipStream_t st) {
  if (dt != MLA_BF16) return gemm_store(h_t, s.K, 0, f32, W_DQ, s.K, 0, false, s, dt, P, cq, s.N, 0, st, MLA_FP32);
  MLA_TRY(gemm(h_t, s.K, 0, f32, W_DQ, s.K, 0, false, s, dt, P, st));
  return hip_status(mla::launch_reduce_store_dual(P, splits_for(s, dt), s.M, s.N, static_cast<float*>(cq),
                                                  static_cast<uint16_t*>(cq16), st),
                    "reduce launch");
}

}  // namespace

extern "C" {

const char* mla_status_str(int32_t s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL: a required pointer is NULL";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE: invalid or inconsistent sizes";
    case MLA_ERR_DTYPE: return "MLA_ERR_DTYPE: unsupported dtype";
    case MLA_ERR_ALIGN: return "MLA_ERR_ALIGN: pointer or row not 16-byte aligned";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace too small";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: no kernel for this shape";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: HIP runtime error";
    default: return "unknown mla_status";
  }
}

const char* mla_last_error(void) { return g_err; }

size_t mla_cache_row_bytes(const mla_dims* dims) {
  if (check_dims(dims) != MLA_OK) return 0;
  return static_cast<size_t>(dims->d_c + dims->d_R) * elem_size(dims->dtype);
}

int32_t mla_decode_kernel(const mla_dims* dims) {
  if (check_dims(dims) != MLA_OK) return 0;
  return mfma_attn(dims) ? 1 : 2;
}

int32_t mla_decode_num_splits(const mla_dims* dims, int32_t B, int32_t max_seq_len, int32_t num_splits) {
  if (check_dims(dims) != MLA_OK || B <= 0 || max_seq_len < 0 || num_splits < 0) return 0;
  if (mfma_attn(dims)) {
    const int s = mfma_splits(num_splits, max_seq_len);
    return mfma_uniform_chunks(B, max_seq_len, s, static_cast<int>(std::min(kMaxMfmaGrid, mfma_grid(B, s))));
  }
  int s = 1, ch = 1;
  attn_plan(dims, B, max_seq_len, num_splits, &s, &ch);
  return s;
}

size_t mla_workspace_bytes(const mla_dims* dims, int32_t B, int32_t max_seq_len, int32_t num_splits) {
  if (check_dims(dims) != MLA_OK || B <= 0 || max_seq_len < 0 || num_splits < 0) return 0;
  size_t w = ws_compress(dims, B);
  w = std::max(w, ws_absorb(dims, B));
  w = std::max(w, ws_attn(dims, B, max_seq_len, num_splits));
  w = std::max(w, ws_out(dims, B));
  w = std::max(w, ws_absorb_pre(dims, B));
  w = std::max(w, ws_out_pre(dims, B));
  return std::max<size_t>(w, 256);
}

mla_status mla_compress_append(const mla_dims* dims, int32_t B, const void* h_t, const void* W_DKV,
                               const void* W_KR, const void* gamma_kv, const int32_t* pos,
                               const mla_cache* cache, void* ws, size_t ws_bytes, void* stream) {
  MLA_TRY(check_dims(dims));
  if (B <= 0) return fail(MLA_ERR_SHAPE, "B must be positive");
  if (!h_t || !W_DKV || !W_KR || !pos || !ws) return fail(MLA_ERR_NULL, "compress_append: NULL pointer");
  MLA_TRY(check_cache(dims, cache));
  for (const void* p : {h_t, W_DKV, W_KR, static_cast<const void*>(pos), static_cast<const void*>(ws)})
    if (!aligned16(p)) return fail(MLA_ERR_ALIGN, "compress_append: pointer not 16-byte aligned");
  if (gamma_kv && !aligned16(gamma_kv)) return fail(MLA_ERR_ALIGN, "gamma_kv not 16-byte aligned");
  const size_t need = ws_compress(dims, B);
  if (ws_bytes < need) return fail(MLA_ERR_WORKSPACE, "compress_append needs %zu bytes", need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int dt = dims->dtype;
  const bool f32 = dt == MLA_FP32;
  char* w = static_cast<char*>(ws);
  const float eps = dims->norm_eps > 0.f ? dims->norm_eps : 1e-6f;
  const int D = dims->d_c + dims->d_R;
  // [c ; k_R] = [W_DKV ; W_KR] h_t as one product when the streaming kernel
  // can take the two weights in one launch
  {
    const GemmShape s{B, D, dims->d, 1};
    mla::GemmArgs g{h_t, dims->d, 0, f32, W_DKV, dims->d, 0, false, s.M, s.N, s.K, s.G, splits_for(s, dt),
                    reinterpret_cast<float*>(w), dt};
    g.W2 = W_KR;
    g.n_split = dims->d_c;
    if (mla::gemm_concat_ok(g)) {
      MLA_TRY(hip_status(mla::launch_gemm(g, st), "gemm launch"));
      const float* P = reinterpret_cast<const float*>(w);
      return hip_status(mla::launch_append(P, g.splits, D, P + dims->d_c, g.splits, D, B, dims->d_c, dims->d_R,
                                           gamma_kv, eps, pos, dims->rope_theta, *cache, dt, st),
                        "append launch");
    }
  }
  float* Pc = reinterpret_cast<float*>(w);
  float* Pr = reinterpret_cast<float*>(w + align_up(part_bytes({B, dims->d_c, dims->d, 1}, dt)));
  const GemmShape sc{B, dims->d_c, dims->d, 1}, sr{B, dims->d_R, dims->d, 1};
  MLA_TRY(gemm(h_t, dims->d, 0, f32, W_DKV, dims->d, 0, false, sc, dt, Pc, st));
  MLA_TRY(gemm(h_t, dims->d, 0, f32, W_KR, dims->d, 0, false, sr, dt, Pr, st));
  MLA_TRY(hip_status(mla::launch_append(Pc, splits_for(sc, dt), dims->d_c, Pr, splits_for(sr, dt), dims->d_R, B,
                                        dims->d_c, dims->d_R, gamma_kv, eps, pos, dims->rope_theta, *cache, dt, st),
                     "append launch"));
  return ok();
}

mla_status mla_absorb_q(const mla_dims* dims, int32_t B, const void* h_t, const void* W_DQ,
                        const void* W_UQ, const void* W_QR, const void* W_UK, const int32_t* pos,
                        void* q, void* ws, size_t ws_bytes, void* stream) {
  MLA_TRY(check_dims(dims));
  if (B <= 0) return fail(MLA_ERR_SHAPE, "B must be positive");
  if (!h_t || !W_UQ || !W_QR || !W_UK || !pos || !q || !ws) return fail(MLA_ERR_NULL, "absorb_q: NULL pointer");
  if ((dims->d_cq > 0) != (W_DQ != nullptr))
    return fail(MLA_ERR_NULL, "absorb_q: W_DQ must be given iff d_cq > 0");
  for (const void* p : {h_t, W_UQ, W_QR, W_UK, static_cast<const void*>(pos), static_cast<const void*>(q),
                        static_cast<const void*>(ws)})
    if (!aligned16(p)) return fail(MLA_ERR_ALIGN, "absorb_q: pointer not 16-byte aligned");
  if (W_DQ && !aligned16(W_DQ)) return fail(MLA_ERR_ALIGN, "absorb_q: W_DQ not 16-byte aligned");
  const size_t need = ws_absorb(dims, B);
  if (ws_bytes < need) return fail(MLA_ERR_WORKSPACE, "absorb_q needs %zu bytes", need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int dt = dims->dtype;
  const size_t es = elem_size(dt);
  const bool f32 = dt == MLA_FP32;
  const int H = dims->H, d_h = dims->d_h, d_R = dims->d_R, d_c = dims->d_c, D = d_c + d_R;
  const int QD = D + d_R;   // query row: [q_lat ; q_R ; the low term of q_R]
  // c_Q and q_C stay in float32: W_QR (the rotary query, which dominates
  // the scores) and W_UK^T read them as two bf16 terms, W_UQ rounds c_Q once
  char* w = static_cast<char*>(ws);
  void* cq = w;
  void* cq16 = w + align_up(static_cast<size_t>(B) * dims->d_cq * sizeof(float));
  void* qC = static_cast<char*>(cq16) + align_up(static_cast<size_t>(B) * dims->d_cq * 2);
  float* P = reinterpret_cast<float*>(static_cast<char*>(qC) +
                                      align_up(static_cast<size_t>(B) * H * d_h * sizeof(float)));
  // c_Q = W_DQ h (or h itself)
  const void* cin = h_t;
  bool cin_f32 = f32;
  const void* cin_uq = h_t;   // W_UQ's activation: c_Q rounded once (bf16 copy)
  bool cin_uq_f32 = f32;
  int qin = dims->d;
  if (dims->d_cq) {
    const GemmShape s{B, dims->d_cq, dims->d, 1};
    MLA_TRY(cq_product(h_t, f32, W_DQ, s, dt, P, cq, cq16, st));
    cin = cq;
    cin_f32 = true;
    cin_uq = f32 ? cq : cq16;
    cin_uq_f32 = f32;
    qin = dims->d_cq;
  }
  // q_C(i) = W_UQ(i) c_Q for all heads at once: W_UQ viewed as [H*d_h][qin]
  {
    const GemmShape s{B, H * d_h, qin, 1};
    MLA_TRY(gemm_store(cin_uq, qin, 0, cin_uq_f32, W_UQ, qin, 0, false, s, dt, P, qC, H * d_h, 0, st, MLA_FP32));
  }
  // q_R(i) = RoPE(W_QR(i) c_Q, pos) into q[b][i][d_c:]
  {
    const GemmShape s{B, H * d_R, qin, 1};
    MLA_TRY(gemm(cin, qin, 0, cin_f32, W_QR, qin, 0, false, s, dt, P, st, /*a_split=*/true));
    void* qr = static_cast<char*>(q) + static_cast<size_t>(d_c) * es;
    MLA_TRY(hip_status(mla::launch_reduce_rope(P, splits_for(s, dt), B, H, d_R, pos, dims->rope_theta, qr,
                                               static_cast<long long>(H) * QD, QD, dt, st),
                       "rope launch"));
  }
  // q_lat(i) = W_UK(i)^T q_C(i): per head g, A_g[b][k] = qC[b][g*d_h + k],
  // W_g(n=c, k) = W_UK[g][k][c] (k-major use of the [d_h][d_c] matrix).
  {
    const GemmShape s{B, d_c, d_h, H};
    MLA_TRY(gemm_store(qC, static_cast<long long>(H) * d_h, d_h, true, W_UK, d_c, static_cast<long long>(d_h) * d_c,
                       true, s, dt, P, q, static_cast<long long>(H) * QD, QD, st, -1, /*a_split=*/true));
  }
  return ok();
}

}  // extern "C"

namespace {

// Dense attention (indices NULL: entry u of sequence b is row u, seq_lens
// rows) or sparse attention (entry u is row indices[b*topk + u], seq_lens
// holds the entry counts, max_seq_len = topk).
mla_status decode_attn_impl(const mla_dims* dims, int32_t B, const void* q, const mla_cache* cache,
                            const int32_t* seq_lens, int32_t max_seq_len, int32_t num_splits, float* o_lat,
                            float* lse, void* ws, size_t ws_bytes, void* stream, const int32_t* indices,
                            int32_t topk, int32_t qpt = 1, AttnTiming tm = AttnTiming{}) {
  MLA_TRY(check_dims(dims));
  if (B <= 0) return fail(MLA_ERR_SHAPE, "B must be positive");
  if (max_seq_len < 0 || num_splits < 0) return fail(MLA_ERR_SHAPE, "negative max_seq_len or num_splits");
  if (!q || !seq_lens || !o_lat) return fail(MLA_ERR_NULL, "decode_attn: NULL pointer");
  MLA_TRY(check_cache(dims, cache));
  if (!indices && !cache->block_table && max_seq_len > cache->capacity)
    return fail(MLA_ERR_SHAPE, "max_seq_len %d exceeds capacity %d", max_seq_len, cache->capacity);
  if (!indices && cache->block_table &&
      static_cast<long long>(max_seq_len) > static_cast<long long>(cache->max_blocks) * cache->block_size)
    return fail(MLA_ERR_SHAPE, "max_seq_len exceeds max_blocks * block_size");
  for (const void* p : {q, static_cast<const void*>(seq_lens), static_cast<const void*>(o_lat)})
    if (!aligned16(p)) return fail(MLA_ERR_ALIGN, "decode_attn: pointer not 16-byte aligned");
  const bool mfma = mfma_attn(dims);
  if (mfma && B > kMaxMfmaBatch) return fail(MLA_ERR_UNSUPPORTED, "decode_attn: B above %d", kMaxMfmaBatch);
  if (mfma && mfma_grid(B, mfma_splits(num_splits, max_seq_len)) > kMaxMfmaGrid)
    return fail(MLA_ERR_UNSUPPORTED, "decode_attn: B * num_splits above %lld", kMaxMfmaGrid);
  int splits = 1, chunk = 1;
  attn_plan(dims, B, max_seq_len, num_splits, &splits, &chunk);
  const size_t need = ws_attn(dims, B, max_seq_len, num_splits);
  if (need && (!ws || ws_bytes < need)) return fail(MLA_ERR_WORKSPACE, "decode_attn needs %zu bytes", need);
  if (need && !aligned16(ws)) return fail(MLA_ERR_ALIGN, "workspace not 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  mla::AttnArgs a{};
  a.q = q;
  a.cache = cache->data;
  a.block_table = cache->block_table;
  a.capacity = cache->capacity;
  a.block_size = cache->block_size;
  a.max_blocks = cache->max_blocks;
  a.seq_lens = seq_lens;
  a.B = B;
  a.H = dims->H;
  a.d_c = dims->d_c;
  a.d_R = dims->d_R;
  a.chunk = chunk;
  a.splits = splits;
  a.scale = softmax_scale(dims);
  a.o_lat = o_lat;
  a.lse = lse;
  a.dtype = dims->dtype;
  a.indices = indices;
  a.topk = topk;
  a.qpt = qpt;
  a.t_start = tm.start;
  a.t_kernel_end = tm.kernel_end;
  a.t_call_end = tm.call_end;
  if (mfma) {
    // the device plans the chunks (balanced when num_splits is 0) and merges them
    const int s = mfma_splits(num_splits, max_seq_len);
    const size_t g = static_cast<size_t>(mfma_grid(B, s));
    char* w = static_cast<char*>(ws);
    a.splits = s;
    a.grid = static_cast<int>(g);
    a.part_o = reinterpret_cast<float*>(w);   // fp16 partials, read as such by the MFMA path
    w += align_up(g * dims->H * dims->d_c * 2);
    a.part_ml = reinterpret_cast<float*>(w);
    w += align_up(g * dims->H * 4 * sizeof(float));
    a.plan_seq = reinterpret_cast<int2*>(w);
    MLA_TRY(hip_status(mla::launch_attn_mfma(a, st), "attention launch"));
    return ok();
  }
  if (splits > 1) {
    a.part_o = static_cast<float*>(ws);
    a.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                         align_up(static_cast<size_t>(B) * splits * dims->H * dims->d_c * sizeof(float)));
  }
  if (max_seq_len == 0) {
    // every sequence is empty: zeros and -inf
    a.splits = 1;
    a.chunk = 1;
  }
  // the general kernel takes the timing events as markers around its launches
  if (tm.start) MLA_TRY(hip_status(hipEventRecord(tm.start, st), "timing event"));
  MLA_TRY(hip_status(mla::launch_attn_generic(a, st), "attention launch"));
  if (tm.kernel_end) MLA_TRY(hip_status(hipEventRecord(tm.kernel_end, st), "timing event"));
  if (a.splits > 1) MLA_TRY(hip_status(mla::launch_attn_combine(a, st), "combine launch"));
  if (tm.call_end) MLA_TRY(hip_status(hipEventRecord(tm.call_end, st), "timing event"));
  return ok();
}

// ---- causal prefill (materialised or absorbed) ----

bool prefill_mfma(const mla_dims* d, const mla_cache* c) {
  return d->dtype == MLA_BF16 && d->d_h == 128 && d->d_R == 64 && d->d_v == 128 &&
         (c->block_table == nullptr || c->block_size >= 8);
}
// Rows the cache stores (every one is expanded), and the transposed values'
// row length and per-sequence column stride (contiguous cache: each
// sequence's columns start on a multiple of 8).
long long cache_store_rows(const mla_cache* c, int B) {
  return c->block_table ? static_cast<long long>(c->n_blocks) * c->block_size
                        : static_cast<long long>(B) * c->capacity;
}
long long vt_seq_stride(const mla_cache* c) { return c->block_table ? 0 : (c->capacity + 7LL) / 8 * 8; }
long long vt_row_len(const mla_cache* c, int B) {
  return c->block_table ? cache_store_rows(c, B) : static_cast<long long>(B) * vt_seq_stride(c);
}

// Partial bytes a gemm_store of this shape needs (none when it stores directly).
size_t store_part_bytes(const GemmShape& s, int dtype, long long lda, long long sAg, bool a_f32, long long ldw,
                        long long sWg, bool w_kn) {
  alignas(16) static const char dummy[16] = {};
  mla::GemmArgs g{dummy, lda, sAg, a_f32, dummy, ldw, sWg, w_kn, s.M, s.N, s.K, s.G, splits_for(s, dtype),
                  nullptr, dtype};
  g.out = const_cast<char*>(dummy);
  return mla::gemm_direct(g) ? 0 : part_bytes(s, dtype);
}

struct PrefillPlan {
  // materialised: expanded keys and transposed values, GEMM partials
  size_t k_bytes = 0, vt_bytes = 0;
  // absorbed: absorbed queries, latent outputs, attention workspace
  size_t qa_bytes = 0, olat_bytes = 0, attn_bytes = 0;
  size_t p_bytes = 0;
  size_t total() const {
    return align_up(k_bytes) + align_up(vt_bytes) + align_up(qa_bytes) + align_up(olat_bytes) +
           align_up(attn_bytes) + align_up(p_bytes);
  }
};

PrefillPlan prefill_plan(const mla_dims* d, int B, int T, int max_seq_len, const mla_cache* c, int algo) {
  PrefillPlan pl;
  const size_t es = elem_size(d->dtype);
  const int H = d->H, D = d->d_c + d->d_R, DQ = d->d_h + d->d_R;
  const bool f32 = d->dtype == MLA_FP32;
  if (algo == MLA_PREFILL_MATERIALIZED) {
    const long long rows = cache_store_rows(c, B);
    pl.k_bytes = static_cast<size_t>(rows) * H * d->d_h * es;
    pl.vt_bytes = static_cast<size_t>(H) * d->d_v * vt_row_len(c, B) * es;
    const GemmShape sk{static_cast<int>(rows), H * d->d_h, d->d_c, 1};
    const bool paged = c->block_table != nullptr;
    const GemmShape sv{H * d->d_v, paged ? static_cast<int>(rows) : c->capacity, d->d_c, paged ? 1 : B};
    pl.p_bytes = std::max(store_part_bytes(sk, d->dtype, D, 0, f32, d->d_c, 0, false),
                          store_part_bytes(sv, d->dtype, d->d_c, 0, f32, D,
                                           paged ? 0 : static_cast<long long>(c->capacity) * D, false));
  } else {
    const long long BT = static_cast<long long>(B) * T;
    pl.qa_bytes = static_cast<size_t>(BT) * H * (D + d->d_R) * es;   // [q_lat ; q_R ; low term]
    pl.olat_bytes = static_cast<size_t>(BT) * H * d->d_c * sizeof(float);
    pl.attn_bytes = ws_attn(d, static_cast<int>(BT), max_seq_len, 0);
    const GemmShape sq{static_cast<int>(BT), d->d_c, d->d_h, H};
    const GemmShape so{static_cast<int>(BT), d->d_v, d->d_c, H};
    pl.p_bytes = std::max(store_part_bytes(sq, d->dtype, static_cast<long long>(H) * DQ, DQ, f32, d->d_c,
                                           static_cast<long long>(d->d_h) * d->d_c, true),
                          store_part_bytes(so, d->dtype, static_cast<long long>(H) * d->d_c, d->d_c, true, d->d_c,
                                           static_cast<long long>(d->d_v) * d->d_c, false));
  }
  return pl;
}

constexpr long long kMaxPrefillRows = 65535LL * 128;   // rows one expansion product takes (128 per z block)

// Why a validated shape has no kernel in this form, or NULL when it has one.
const char* prefill_unfit(const mla_dims* d, int B, int T, const mla_cache* c, int algo) {
  if (algo == MLA_PREFILL_MATERIALIZED) {
    if (cache_store_rows(c, B) > kMaxPrefillRows || static_cast<long long>(d->H) * d->d_v > kMaxPrefillRows)
      return "prefill: cache too large to expand in one product";
    if (!prefill_mfma(d, c) && d->d_v > 1024) return "prefill: d_v above 1024";
  } else {
    const long long BT = static_cast<long long>(B) * T;
    static_assert(kMaxMfmaBatch == 32768, "the message below names the limit");
    if (mfma_attn(d) && BT > kMaxMfmaBatch) return "prefill (absorbed): B * T above 32768";
    if (BT > kMaxPrefillRows) return "prefill: B * T too large";
  }
  return nullptr;
}

// MLA_PREFILL_AUTO. Costs fitted to the prefill sweep on MI355X (V3 widths,
// 4 sequences of 4096 rows, T = 1 .. 1024): the absorbed form costs about
// 0.30 ns per attended row (row, token) and the materialised form 0.10 ns per
// attended row plus 76 ns per stored row (the expansion). The linear fit puts
// the two equal near 380 attended rows per stored row; measured, the absorbed
// form is 7% faster at 366 and the two are within 0.4% at 424, so the absorbed
// form is taken below 400. Attended rows are bounded from T and max_seq_len
// (every sequence taken at max_seq_len); a form with no kernel for the shape
// yields to the other.
constexpr double kPrefillAutoRatio = 400.0;
int resolve_prefill_algo(const mla_dims* d, int B, int T, int max_seq_len, const mla_cache* c) {
  const double L = max_seq_len, t = T;
  const double per_seq = T <= max_seq_len ? t * L - t * (t - 1.0) / 2.0 : L * (L + 1.0) / 2.0;
  const double attended = static_cast<double>(B) * per_seq;
  const double stored = static_cast<double>(cache_store_rows(c, B));
  int pick = attended < kPrefillAutoRatio * stored ? MLA_PREFILL_ABSORBED : MLA_PREFILL_MATERIALIZED;
  if (prefill_unfit(d, B, T, c, pick))
    pick = pick == MLA_PREFILL_ABSORBED ? MLA_PREFILL_MATERIALIZED : MLA_PREFILL_ABSORBED;
  return pick;
}

// Validates the arguments and resolves MLA_PREFILL_AUTO in *algo.
mla_status check_prefill_sizes(const mla_dims* d, int B, int T, int max_seq_len, const mla_cache* c, int* algo) {
  if (B <= 0 || T <= 0) return fail(MLA_ERR_SHAPE, "prefill: B and T must be positive");
  if (max_seq_len < 0) return fail(MLA_ERR_SHAPE, "prefill: negative max_seq_len");
  if (*algo != MLA_PREFILL_MATERIALIZED && *algo != MLA_PREFILL_ABSORBED && *algo != MLA_PREFILL_AUTO)
    return fail(MLA_ERR_SHAPE, "prefill: unknown algorithm %d", *algo);
  MLA_TRY(check_cache(d, c));
  if (!c->block_table && max_seq_len > c->capacity)
    return fail(MLA_ERR_SHAPE, "max_seq_len %d exceeds capacity %d", max_seq_len, c->capacity);
  if (c->block_table && static_cast<long long>(max_seq_len) > static_cast<long long>(c->max_blocks) * c->block_size)
    return fail(MLA_ERR_SHAPE, "max_seq_len exceeds max_blocks * block_size");
  if (*algo == MLA_PREFILL_AUTO) *algo = resolve_prefill_algo(d, B, T, max_seq_len, c);
  if (const char* why = prefill_unfit(d, B, T, c, *algo)) return fail(MLA_ERR_UNSUPPORTED, "%s", why);
  return MLA_OK;
}

mla_status prefill_materialized(const mla_dims* d, int B, int T, const void* q, const mla_cache* c,
                                const int32_t* seq_lens, const void* W_UK, const void* W_UV, void* o, float* lse,
                                const PrefillPlan& pl, char* w, hipStream_t st) {
  const int dt = d->dtype;
  const bool f32 = dt == MLA_FP32;
  const int H = d->H, D = d->d_c + d->d_R;
  void* Kx = w;
  w += align_up(pl.k_bytes);
  void* Vt = w;
  w += align_up(pl.vt_bytes);
  float* P = reinterpret_cast<float*>(w);
  const long long rows = cache_store_rows(c, B);
  const bool paged = c->block_table != nullptr;
  const long long vt_ld = vt_row_len(c, B), vt_seq = vt_seq_stride(c);
  // Expansion products: the tall kernel when it takes the shape, else the
  // general GEMM with its own store.
  auto expand = [&](const void* Am, long long lda, long long sAg, const void* Wm, long long ldw, long long sWg,
                    const GemmShape& s, void* out, long long ldo, long long sOg) -> mla_status {
    mla::GemmArgs g{Am, lda, sAg, f32, Wm, ldw, sWg, false, s.M, s.N, s.K, s.G, 1, P, dt};
    g.out = out;
    g.ldo = ldo;
    g.sOg = sOg;
    g.out_dtype = dt;
    if (mla::gemm_tall_ok(g)) return hip_status(mla::launch_gemm_tall(g, st), "gemm launch");
    return gemm_store(Am, lda, sAg, f32, Wm, ldw, sWg, false, s, dt, P, out, ldo, sOg, st);
  };
  // K[row][i*d_h + k] = (W_UK(i) c_row)[k] for every stored row
  MLA_TRY(expand(c->data, D, 0, W_UK, d->d_c, 0, GemmShape{static_cast<int>(rows), H * d->d_h, d->d_c, 1}, Kx,
                 static_cast<long long>(H) * d->d_h, 0));
  // Vt[i*d_v + j][col] = (W_UV(i) c_row)[j]: W_UV times the rows, per sequence
  // (contiguous) or over the whole pool (paged)
  MLA_TRY(expand(W_UV, d->d_c, 0, c->data, D, paged ? 0 : static_cast<long long>(c->capacity) * D,
                 GemmShape{H * d->d_v, paged ? static_cast<int>(rows) : c->capacity, d->d_c, paged ? 1 : B}, Vt,
                 vt_ld, paged ? 0 : vt_seq));
  mla::PrefillArgs a{};
  a.q = q;
  a.K = Kx;
  a.Vt = Vt;
  a.vt_ld = vt_ld;
  a.vt_seq = vt_seq;
  a.cache = c->data;
  a.block_table = c->block_table;
  a.capacity = c->capacity;
  a.block_size = c->block_size;
  a.max_blocks = c->max_blocks;
  a.seq_lens = seq_lens;
  a.B = B;
  a.T = T;
  a.H = H;
  a.d_h = d->d_h;
  a.d_v = d->d_v;
  a.d_c = d->d_c;
  a.d_R = d->d_R;
  a.scale = softmax_scale(d);
  a.o = o;
  a.lse = lse;
  a.dtype = dt;
  if (prefill_mfma(d, c)) return hip_status(mla::launch_prefill_mfma(a, st), "prefill launch");
  return hip_status(mla::launch_prefill_generic(a, st), "prefill launch");
}

mla_status prefill_absorbed(const mla_dims* d, int B, int T, const void* q, const mla_cache* c,
                            const int32_t* seq_lens, int max_seq_len, const void* W_UK, const void* W_UV, void* o,
                            float* lse, const PrefillPlan& pl, char* w, hipStream_t st) {
  const int dt = d->dtype;
  const size_t es = elem_size(dt);
  const bool f32 = dt == MLA_FP32;
  const int H = d->H, D = d->d_c + d->d_R, DQ = d->d_h + d->d_R;
  const int QD = D + d->d_R;   // absorbed query row: [q_lat ; q_R ; zero low term]
  const int BT = B * T;
  void* qa = w;
  w += align_up(pl.qa_bytes);
  float* olat = reinterpret_cast<float*>(w);
  w += align_up(pl.olat_bytes);
  void* aw = w;
  w += align_up(pl.attn_bytes);
  float* P = reinterpret_cast<float*>(w);
  // q_lat(t, i) = W_UK(i)^T q_C(t, i) into qa[t][i][0:d_c]
  {
    const GemmShape s{BT, d->d_c, d->d_h, H};
    MLA_TRY(gemm_store(q, static_cast<long long>(H) * DQ, DQ, f32, W_UK, d->d_c, static_cast<long long>(d->d_h) * d->d_c,
                       true, s, dt, P, qa, static_cast<long long>(H) * QD, QD, st));
  }
  // q_R(t, i) beside it (given in the storage type: its second term is zero)
  MLA_TRY(hip_status(mla::launch_rope_query_copy(q, DQ, d->d_h, qa, QD, d->d_c, d->d_R,
                                                 static_cast<long long>(BT) * H, dt, st),
                     "rotary query copy"));
  // token t of sequence b attends rows 0 .. seq_lens[b] - T + t
  MLA_TRY(decode_attn_impl(d, BT, qa, c, seq_lens, max_seq_len, 0, olat, lse, aw, pl.attn_bytes, st, nullptr, 0, T));
  // o(t, i) = W_UV(i) o_lat(t, i)
  const GemmShape s{BT, d->d_v, d->d_c, H};
  return gemm_store(olat, static_cast<long long>(H) * d->d_c, d->d_c, true, W_UV, d->d_c,
                    static_cast<long long>(d->d_v) * d->d_c, false, s, dt, P, o, static_cast<long long>(H) * d->d_v,
                    d->d_v, st);
}

}  // namespace

extern "C" {

size_t mla_prefill_workspace_bytes(const mla_dims* dims, int32_t B, int32_t T, int32_t max_seq_len,
                                   const mla_cache* cache, int32_t algo) {
  if (check_dims(dims) != MLA_OK || !cache) return 0;
  if (check_prefill_sizes(dims, B, T, max_seq_len, cache, &algo) != MLA_OK) return 0;
  return prefill_plan(dims, B, T, max_seq_len, cache, algo).total();
}

int32_t mla_prefill_choose(const mla_dims* dims, int32_t B, int32_t T, int32_t max_seq_len,
                           const mla_cache* cache) {
  if (check_dims(dims) != MLA_OK || !cache) return -1;
  int32_t algo = MLA_PREFILL_AUTO;
  if (check_prefill_sizes(dims, B, T, max_seq_len, cache, &algo) != MLA_OK) return -1;
  return algo;
}

mla_status mla_prefill_attn(const mla_dims* dims, int32_t B, int32_t T, const void* q, const mla_cache* cache,
                            const int32_t* seq_lens, int32_t max_seq_len, const void* W_UK, const void* W_UV,
                            int32_t algo, void* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  MLA_TRY(check_dims(dims));
  if (!q || !cache || !seq_lens || !W_UK || !W_UV || !o || !ws) return fail(MLA_ERR_NULL, "prefill: NULL pointer");
  MLA_TRY(check_prefill_sizes(dims, B, T, max_seq_len, cache, &algo));
  for (const void* p : {q, static_cast<const void*>(seq_lens), W_UK, W_UV, static_cast<const void*>(o),
                        static_cast<const void*>(ws)})
    if (!aligned16(p)) return fail(MLA_ERR_ALIGN, "prefill: pointer not 16-byte aligned");
  if (lse && !aligned16(lse)) return fail(MLA_ERR_ALIGN, "prefill: lse not 16-byte aligned");
  const PrefillPlan pl = prefill_plan(dims, B, T, max_seq_len, cache, algo);
  if (ws_bytes < pl.total()) return fail(MLA_ERR_WORKSPACE, "prefill needs %zu bytes", pl.total());
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  if (algo == MLA_PREFILL_MATERIALIZED)
    return prefill_materialized(dims, B, T, q, cache, seq_lens, W_UK, W_UV, o, lse, pl, w, st);
  return prefill_absorbed(dims, B, T, q, cache, seq_lens, max_seq_len, W_UK, W_UV, o, lse, pl, w, st);
}

mla_status mla_decode_attn(const mla_dims* dims, int32_t B, const void* q, const mla_cache* cache,
                           const int32_t* seq_lens, int32_t max_seq_len, int32_t num_splits, float* o_lat,
                           float* lse, void* ws, size_t ws_bytes, void* stream) {
  const AttnTiming tm = take_attn_timing();
  return decode_attn_impl(dims, B, q, cache, seq_lens, max_seq_len, num_splits, o_lat, lse, ws, ws_bytes, stream,
                          nullptr, 0, 1, tm);
}

mla_status mla_time_next_attn(void* kernel_start, void* kernel_end, void* call_end) {
  g_attn_timing.start = static_cast<hipEvent_t>(kernel_start);
  g_attn_timing.kernel_end = static_cast<hipEvent_t>(kernel_end);
  g_attn_timing.call_end = static_cast<hipEvent_t>(call_end);
  return ok();
}

mla_status mla_decode_attn_sparse(const mla_dims* dims, int32_t B, const void* q, const mla_cache* cache,
                                  const int32_t* indices, int32_t topk, const int32_t* counts, int32_t num_splits,
                                  float* o_lat, float* lse, void* ws, size_t ws_bytes, void* stream) {
  const AttnTiming tm = take_attn_timing();
  if (topk <= 0) return fail(MLA_ERR_SHAPE, "decode_attn_sparse: topk must be positive");
  if (!indices || !counts) return fail(MLA_ERR_NULL, "decode_attn_sparse: NULL indices or counts");
  if ((reinterpret_cast<uintptr_t>(indices) | reinterpret_cast<uintptr_t>(counts)) & 3)
    return fail(MLA_ERR_ALIGN, "decode_attn_sparse: indices and counts must be 4-byte aligned");
  return decode_attn_impl(dims, B, q, cache, counts, topk, num_splits, o_lat, lse, ws, ws_bytes, stream, indices,
                          topk, 1, tm);
}

mla_status mla_check_indices(const mla_dims* dims, int32_t B, const mla_cache* cache, const int32_t* pos,
                             const int32_t* seq_lens, int32_t max_seq_len, const int32_t* block_table,
                             const int32_t* indices, int32_t topk, const int32_t* counts) {
  MLA_TRY(check_dims(dims));
  if (B <= 0) return fail(MLA_ERR_SHAPE, "B must be positive");
  MLA_TRY(check_cache(dims, cache));
  const bool paged = cache->block_table != nullptr;
  if (paged && !block_table && (pos || seq_lens || indices))
    return fail(MLA_ERR_NULL, "check_indices: a paged cache needs the host copy of its block table");
  if ((indices == nullptr) != (counts == nullptr))
    return fail(MLA_ERR_NULL, "check_indices: indices and counts go together");
  if (indices && topk <= 0) return fail(MLA_ERR_SHAPE, "check_indices: topk must be positive");
  const long long bs = paged ? cache->block_size : 0;
  const long long rows_max = paged ? static_cast<long long>(cache->max_blocks) * bs : cache->capacity;
  // Block entry of row u of sequence b (paged): -1 when the entry is outside the pool.
  auto block_of = [&](int b, long long u) -> long long {
    const long long e = block_table[static_cast<long long>(b) * cache->max_blocks + u / bs];
    return (e >= 0 && e < cache->n_blocks) ? e : -1;
  };
  if (pos) {
    for (int b = 0; b < B; ++b) {
      const long long t = pos[b];
      if (t < 0 || t >= rows_max)
        return fail(MLA_ERR_SHAPE, "check_indices: pos[%d] = %lld outside the sequence's %lld rows", b, t, rows_max);
      if (paged && block_of(b, t) < 0)
        return fail(MLA_ERR_SHAPE, "check_indices: pos[%d] = %lld falls in block-table entry %lld, not a block of "
                    "the pool", b, t, t / bs);
    }
    if (paged) {
      // two sequences appending into one cache slot would race
      std::vector<long long> slots(B);
      for (int b = 0; b < B; ++b) slots[b] = block_of(b, pos[b]) * bs + pos[b] % bs;
      std::vector<long long> sorted(slots);
      std::sort(sorted.begin(), sorted.end());
      for (int i = 1; i < B; ++i)
        if (sorted[i] == sorted[i - 1]) {
          int b0 = -1, b1 = -1;
          for (int b = 0; b < B; ++b)
            if (slots[b] == sorted[i]) (b0 < 0 ? b0 : b1) = b;
          return fail(MLA_ERR_SHAPE, "check_indices: sequences %d and %d append into the same cache slot", b0, b1);
        }
    }
  }
  if (seq_lens) {
    if (max_seq_len < 0) return fail(MLA_ERR_SHAPE, "check_indices: negative max_seq_len");
    for (int b = 0; b < B; ++b) {
      const long long L = seq_lens[b];
      if (L < 0 || L > max_seq_len)
        return fail(MLA_ERR_SHAPE, "check_indices: seq_lens[%d] = %lld outside [0, max_seq_len = %d]", b, L,
                    max_seq_len);
      if (L > rows_max)
        return fail(MLA_ERR_SHAPE, "check_indices: seq_lens[%d] = %lld exceeds the sequence's %lld rows", b, L,
                    rows_max);
      if (paged)
        for (long long u = 0; u < L; u += bs)
          if (block_of(b, u) < 0)
            return fail(MLA_ERR_SHAPE, "check_indices: sequence %d reads rows of block-table entry %lld, not a "
                        "block of the pool", b, u / bs);
    }
  }
  if (indices) {
    for (int b = 0; b < B; ++b) {
      const long long n = counts[b];
      if (n < 0 || n > topk)
        return fail(MLA_ERR_SHAPE, "check_indices: counts[%d] = %lld outside [0, topk = %d]", b, n, topk);
      const long long lim = seq_lens ? std::min<long long>(seq_lens[b], rows_max) : rows_max;
      for (long long j = 0; j < n; ++j) {
        const long long u = indices[static_cast<long long>(b) * topk + j];
        if (u < 0 || u >= lim)
          return fail(MLA_ERR_SHAPE, "check_indices: indices[%d][%lld] = %lld outside [0, %lld)", b, j, u, lim);
        if (paged && block_of(b, u) < 0)
          return fail(MLA_ERR_SHAPE, "check_indices: indices[%d][%lld] = %lld falls in block-table entry %lld, not "
                      "a block of the pool", b, j, u, u / bs);
      }
    }
  }
  return ok();
}

mla_status mla_precompose(const mla_dims* dims, const void* W_UQ, const void* W_UK, const void* W_UV,
                          const void* W_O, void* W_QK, void* W_OV, void* stream) {
  MLA_TRY(check_dims(dims));
  if (!W_UQ || !W_UK || !W_QK) return fail(MLA_ERR_NULL, "precompose: NULL W_UQ, W_UK or W_QK");
  if ((W_OV != nullptr) != (W_UV != nullptr && W_O != nullptr) || ((W_UV == nullptr) != (W_O == nullptr)))
    return fail(MLA_ERR_NULL, "precompose: W_UV, W_O and W_OV must all be given or all be NULL");
  for (const void* p : {W_UQ, W_UK, static_cast<const void*>(W_QK), W_UV, W_O, static_cast<const void*>(W_OV)})
    if (p && !aligned16(p)) return fail(MLA_ERR_ALIGN, "precompose: pointer not 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int dt = dims->dtype;
  const int H = dims->H, d_h = dims->d_h, d_v = dims->d_v, d_c = dims->d_c;
  const int qin = dims->d_cq ? dims->d_cq : dims->d;
  // W_QK(i)[m][n] = sum_k W_UK(i)[k][m] W_UQ(i)[k][n]
  MLA_TRY(hip_status(mla::launch_compose(W_UK, static_cast<long long>(d_h) * d_c, d_c, 1, W_UQ,
                                         static_cast<long long>(d_h) * qin, qin, W_QK,
                                         static_cast<long long>(d_c) * qin, qin, H, d_c, qin, d_h, dt, st),
                     "compose launch"));
  if (W_OV) {
    // W_OV[r][i*d_c + n] = sum_k W_O[r][i*d_v + k] W_UV(i)[k][n]
    MLA_TRY(hip_status(mla::launch_compose(W_O, d_v, 1, static_cast<long long>(H) * d_v, W_UV,
                                           static_cast<long long>(d_v) * d_c, d_c, W_OV, d_c,
                                           static_cast<long long>(H) * d_c, H, dims->d, d_c, d_v, dt, st),
                       "compose launch"));
  }
  return ok();
}

mla_status mla_absorb_q_precomposed(const mla_dims* dims, int32_t B, const void* h_t, const void* W_DQ,
                                    const void* W_QK, const void* W_QR, const int32_t* pos, void* q, void* ws,
                                    size_t ws_bytes, void* stream) {
  MLA_TRY(check_dims(dims));
  if (B <= 0) return fail(MLA_ERR_SHAPE, "B must be positive");
  if (!h_t || !W_QK || !W_QR || !pos || !q || !ws) return fail(MLA_ERR_NULL, "absorb_q_precomposed: NULL pointer");
  if ((dims->d_cq != 0) != (W_DQ != nullptr))
    return fail(MLA_ERR_NULL, "absorb_q_precomposed: W_DQ must be given iff d_cq > 0");
  for (const void* p : {h_t, W_QK, W_QR, static_cast<const void*>(pos), static_cast<const void*>(q),
                        static_cast<const void*>(ws)})
    if (!aligned16(p)) return fail(MLA_ERR_ALIGN, "absorb_q_precomposed: pointer not 16-byte aligned");
  if (W_DQ && !aligned16(W_DQ)) return fail(MLA_ERR_ALIGN, "absorb_q_precomposed: W_DQ not 16-byte aligned");
  const size_t need = ws_absorb_pre(dims, B);
  if (ws_bytes < need) return fail(MLA_ERR_WORKSPACE, "absorb_q_precomposed needs %zu bytes", need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int dt = dims->dtype;
  const size_t es = elem_size(dt);
  const bool f32 = dt == MLA_FP32;
  const int H = dims->H, d_R = dims->d_R, d_c = dims->d_c, D = d_c + d_R;
  const int QD = D + d_R;   // query row: [q_lat ; q_R ; the low term of q_R]
  char* w = static_cast<char*>(ws);
  void* cq = w;   // float32 and a bf16 copy, as in mla_absorb_q
  void* cq16 = w + align_up(static_cast<size_t>(B) * dims->d_cq * sizeof(float));
  float* P = reinterpret_cast<float*>(static_cast<char*>(cq16) + align_up(static_cast<size_t>(B) * dims->d_cq * 2));
  const void* cin = h_t;
  bool cin_f32 = f32;
  const void* cin_qk = h_t;   // W_QK's activation: c_Q rounded once
  bool cin_qk_f32 = f32;
  int qin = dims->d;
  if (dims->d_cq) {
    const GemmShape s{B, dims->d_cq, dims->d, 1};
    MLA_TRY(cq_product(h_t, f32, W_DQ, s, dt, P, cq, cq16, st));
    cin = cq;
    cin_f32 = true;
    cin_qk = f32 ? cq : cq16;
    cin_qk_f32 = f32;
    qin = dims->d_cq;
  }
  // q_lat(i) = W_QK(i) c_Q: one activation row per sequence shared by all heads
  {
    const GemmShape s{B, d_c, qin, H};
    MLA_TRY(gemm_store(cin_qk, qin, 0, cin_qk_f32, W_QK, qin, static_cast<long long>(d_c) * qin, false, s, dt, P, q,
                       static_cast<long long>(H) * QD, QD, st));
  }
  // q_R(i) = RoPE(W_QR(i) c_Q, pos), as in mla_absorb_q
  {
    const GemmShape s{B, H * d_R, qin, 1};
    MLA_TRY(gemm(cin, qin, 0, cin_f32, W_QR, qin, 0, false, s, dt, P, st, /*a_split=*/true));
    void* qr = static_cast<char*>(q) + static_cast<size_t>(d_c) * es;
    MLA_TRY(hip_status(mla::launch_reduce_rope(P, splits_for(s, dt), B, H, d_R, pos, dims->rope_theta, qr,
                                               static_cast<long long>(H) * QD, QD, dt, st),
                       "rope launch"));
  }
  return ok();
}

mla_status mla_out_proj_precomposed(const mla_dims* dims, int32_t B, const float* o_lat, const void* W_OV, void* out,
                                    void* ws, size_t ws_bytes, void* stream) {
  MLA_TRY(check_dims(dims));
  if (B <= 0) return fail(MLA_ERR_SHAPE, "B must be positive");
  if (!o_lat || !W_OV || !out || !ws) return fail(MLA_ERR_NULL, "out_proj_precomposed: NULL pointer");
  for (const void* p : {static_cast<const void*>(o_lat), W_OV, static_cast<const void*>(out),
                        static_cast<const void*>(ws)})
    if (!aligned16(p)) return fail(MLA_ERR_ALIGN, "out_proj_precomposed: pointer not 16-byte aligned");
  const size_t need = ws_out_pre(dims, B);
  if (ws_bytes < need) return fail(MLA_ERR_WORKSPACE, "out_proj_precomposed needs %zu bytes", need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int dt = dims->dtype;
  const long long K = static_cast<long long>(dims->H) * dims->d_c;
  // out(b) = W_OV o_lat(b) over all heads' latents at once
  const GemmShape s{B, dims->d, static_cast<int>(K), 1};
  return gemm_store(o_lat, K, 0, true, W_OV, K, 0, false, s, dt, static_cast<float*>(ws), out, dims->d, 0, st);
}

mla_status mla_out_proj(const mla_dims* dims, int32_t B, const float* o_lat, const void* W_UV, const void* W_O,
                        void* o_heads, void* out, void* ws, size_t ws_bytes, void* stream) {
  MLA_TRY(check_dims(dims));
  if (B <= 0) return fail(MLA_ERR_SHAPE, "B must be positive");
  if (!o_lat || !W_UV || !o_heads || !ws) return fail(MLA_ERR_NULL, "out_proj: NULL pointer");
  if ((W_O == nullptr) != (out == nullptr)) return fail(MLA_ERR_NULL, "out_proj: W_O and out must both be given or both NULL");
  for (const void* p : {static_cast<const void*>(o_lat), W_UV, static_cast<const void*>(o_heads),
                        static_cast<const void*>(ws)})
    if (!aligned16(p)) return fail(MLA_ERR_ALIGN, "out_proj: pointer not 16-byte aligned");
  if (W_O && (!aligned16(W_O) || !aligned16(out))) return fail(MLA_ERR_ALIGN, "out_proj: W_O/out not aligned");
  const size_t need = ws_out(dims, B);
  if (ws_bytes < need) return fail(MLA_ERR_WORKSPACE, "out_proj needs %zu bytes", need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int dt = dims->dtype;
  const bool f32 = dt == MLA_FP32;
  const int H = dims->H, d_v = dims->d_v, d_c = dims->d_c;
  float* P = static_cast<float*>(ws);
  {
    // o_heads(b,i) = W_UV(i) o_lat(b,i): per head g, A_g[b][c] = o_lat[b][g][c]
    const GemmShape s{B, d_v, d_c, H};
    MLA_TRY(gemm_store(o_lat, static_cast<long long>(H) * d_c, d_c, true, W_UV, d_c, static_cast<long long>(d_v) * d_c,
                       false, s, dt, P, o_heads, static_cast<long long>(H) * d_v, d_v, st));
  }
  if (W_O) {
    const GemmShape s{B, dims->d, H * d_v, 1};
    MLA_TRY(gemm_store(o_heads, static_cast<long long>(H) * d_v, 0, f32, W_O, static_cast<long long>(H) * d_v, 0,
                       false, s, dt, P, out, dims->d, 0, st));
  }
  return ok();
}

}  // extern "C"

// ---- allocation-free decode attention ----
//
// Scratch for mla_decode_attn_noalloc: one fixed array per device, held by the
// loaded code object until the process ends. Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the device
// symbol): the first call on each device looks its device address up with
// hipGetSymbolAddress, and every later use goes through that address.
namespace {

__device__ __align__(256) char scratch[MLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up once per device).
mla_status scratch_address(void** out) {
  int dev = 0;
  MLA_TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices) return fail(MLA_ERR_UNSUPPORTED, "device index %d above %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    MLA_TRY(hip_status(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
    if (!ptr) return fail(MLA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

}  // namespace

extern "C" mla_status mla_decode_attn_noalloc(const mla_dims* dims, int32_t B, const void* q, const mla_cache* cache,
                                              const int32_t* seq_lens, int32_t max_seq_len, int32_t num_splits,
                                              float* o_lat, float* lse, void* stream) {
  const AttnTiming tm = take_attn_timing();
  MLA_TRY(check_dims(dims));
  if (B <= 0) return fail(MLA_ERR_SHAPE, "B must be positive");
  if (max_seq_len < 0 || num_splits < 0) return fail(MLA_ERR_SHAPE, "negative max_seq_len or num_splits");
  const size_t need = ws_attn(dims, B, max_seq_len, num_splits);
  if (need > MLA_NOALLOC_SCRATCH_BYTES)
    return fail(MLA_ERR_WORKSPACE, "decode_attn_noalloc needs %zu bytes of scratch, above the %zu-byte static array "
                "(fewer sequences or splits per call)", need, static_cast<size_t>(MLA_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  MLA_TRY(scratch_address(&ws));
  return decode_attn_impl(dims, B, q, cache, seq_lens, max_seq_len, num_splits, o_lat, lse, ws,
                          MLA_NOALLOC_SCRATCH_BYTES, stream, nullptr, 0, 1, tm);
}
