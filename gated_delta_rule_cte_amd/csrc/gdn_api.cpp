// libgdn C ABI (include/gdn.h): argument validation and kernel dispatch.
//
// Every check runs before the first HIP call, so a rejected call launches
// nothing and touches no output; the device check comes last.  The library
// holds no device memory and never synchronises.
#include "gdn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "gdn_launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return GDN_OK;
}

struct Span {
  const char* name;
  const void* p;
  size_t bytes;
};

bool overlaps(const Span& a, const Span& b) {
  if (a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// NULL and 16-byte alignment checks for the non-empty spans
int check_ptrs(const std::vector<Span>& spans) {
  for (const Span& s : spans) {
    if (s.bytes == 0) continue;
    if (!s.p) return fail(GDN_ERR_NULL, "%s is NULL", s.name);
  }
  for (const Span& s : spans) {
    if (s.bytes == 0) continue;
    if (reinterpret_cast<uintptr_t>(s.p) & 15u) return fail(GDN_ERR_ALIGN, "%s is not 16-byte aligned", s.name);
  }
  return GDN_OK;
}

// `out` must not overlap any span in `ins` except those listed as exact aliases
int check_disjoint(const Span& out, const std::vector<Span>& ins, const void* allowed_alias = nullptr) {
  for (const Span& s : ins) {
    if (!overlaps(out, s)) continue;
    if (allowed_alias && s.p == allowed_alias && out.p == allowed_alias && s.bytes == out.bytes) continue;
    return fail(GDN_ERR_ALIAS, "%s overlaps %s", out.name, s.name);
  }
  return GDN_OK;
}

bool head_dim_ok(int d) { return d >= 8 && d <= GDN_MAX_HEAD_DIM && d % 8 == 0; }

std::mutex g_dev_mu;
std::vector<int> g_dev_state;  // per device: 0 unknown, 1 gfx950, -1 other

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(GDN_ERR_DEVICE, "no HIP device is available");
  }
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if ((int)g_dev_state.size() <= dev) g_dev_state.resize(dev + 1, 0);
  if (g_dev_state[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(GDN_ERR_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
    }
    g_dev_state[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    if (g_dev_state[dev] < 0) return fail(GDN_ERR_DEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  }
  if (g_dev_state[dev] < 0) return fail(GDN_ERR_DEVICE, "device %d is not gfx950", dev);
  return GDN_OK;
}

int launched(hipError_t e) {
  if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t esize(int dtype) { return dtype == GDN_BF16 ? 2 : 4; }

}  // namespace

namespace gdn {
int set_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}
}  // namespace gdn

extern "C" {

int gdn_version(void) { return 100; }

const char* gdn_last_error(void) { return g_last_error.c_str(); }

const char* gdn_status_string(int status) {
  switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_NULL: return "GDN_ERR_NULL";
    case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE";
    case GDN_ERR_DTYPE: return "GDN_ERR_DTYPE";
    case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN";
    case GDN_ERR_ALIAS: return "GDN_ERR_ALIAS";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_LAUNCH: return "GDN_ERR_LAUNCH";
    case GDN_ERR_DEVICE: return "GDN_ERR_DEVICE";
    default: return "GDN_ERR_UNKNOWN";
  }
}

// ------------------------------------------------------------------ gdn_cte
size_t gdn_cte_workspace_size(int B, int Hk, int Hv, int S, int Dk, int Dv, int dtype) {
  (void)Hk;
  (void)Dk;
  (void)Dv;
  if (B <= 0 || Hv <= 0 || S <= 0 || (dtype != GDN_F32 && dtype != GDN_BF16)) return 0;
  return gdn::cte_workspace_bytes(B, Hv, S, dtype);
}

int gdn_cte(const void* query, const void* key, const void* value, const float* g_log,
            const float* beta, float scale, float* recurrent_state, int has_initial_state,
            void* out, int B, int Hk, int Hv, int S, int Dk, int Dv, int dtype, int algorithm,
            void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != GDN_F32 && dtype != GDN_BF16) return fail(GDN_ERR_DTYPE, "dtype %d is not GDN_F32 or GDN_BF16", dtype);
  if (algorithm != GDN_CTE_ALGO_DEFAULT && algorithm != GDN_CTE_ALGO_NEUMANN)
    return fail(GDN_ERR_UNSUPPORTED, "algorithm %d is not implemented (GDN_CTE_ALGO_DEFAULT or GDN_CTE_ALGO_NEUMANN)",
                algorithm);
  if (B < 0 || S < 0) return fail(GDN_ERR_SHAPE, "B=%d and S=%d must be >= 0", B, S);
  if (Hk < 1 || Hv < 1 || Hv % Hk != 0) return fail(GDN_ERR_SHAPE, "Hv=%d must be a positive multiple of Hk=%d", Hv, Hk);
  if (!head_dim_ok(Dk) || !head_dim_ok(Dv))
    return fail(GDN_ERR_SHAPE, "Dk=%d, Dv=%d must be multiples of 8 in [8, %d]", Dk, Dv, GDN_MAX_HEAD_DIM);
  if ((long long)B * Hv * ((Dv + 15) / 16) > 0x7fffffffLL) return fail(GDN_ERR_SHAPE, "B*Hv too large");
  const size_t es = esize(dtype);
  // per-head extents are addressed with 32-bit buffer offsets below 2^31
  if ((size_t)S * 256 * es >= ((size_t)1 << 31))
    return fail(GDN_ERR_SHAPE, "S=%d is too long for one call (per-head data must stay below 2 GiB)", S);
  const size_t nqk = (size_t)B * Hk * S * Dk * es, nv = (size_t)B * Hv * S * Dv * es;
  const size_t ng = (size_t)B * Hv * S * 4, ns = (size_t)B * Hv * Dk * Dv * 4;
  const Span q{"query", query, nqk}, k{"key", key, nqk}, v{"value", value, nv}, g{"g_log", g_log, ng},
      be{"beta", beta, ng}, st{"recurrent_state", recurrent_state, ns}, o{"out", out, nv};
  if (int r = check_ptrs({q, k, v, g, be, st, o})) return r;
  if (int r = check_disjoint(o, {q, k, v, g, be, st})) return r;
  if (int r = check_disjoint(st, {q, k, v, g, be})) return r;
  if ((size_t)B * Hv == 0) return ok();
  const size_t need = gdn_cte_workspace_size(B, Hk, Hv, S, Dk, Dv, dtype);
  if (need > 0) {
    if (!workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL (%zu bytes required)", need);
    if (workspace_bytes < need)
      return fail(GDN_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
      return fail(GDN_ERR_ALIGN, "workspace is not 256-byte aligned");
    const Span ws{"workspace", workspace, need};
    if (int r = check_disjoint(ws, {q, k, v, g, be, st, o})) return r;
  }
  if (int r = check_device()) return r;
  gdn::CteParams p{};
  p.q = query; p.k = key; p.v = value; p.g = g_log; p.beta = beta;
  p.state = recurrent_state; p.out = out;
  p.B = B; p.Hk = Hk; p.Hv = Hv; p.S = S; p.Dk = Dk; p.Dv = Dv;
  p.has_initial_state = has_initial_state ? 1 : 0;
  p.scale = scale;
  p.algo = algorithm;
  p.ws = workspace;
  return launched(gdn::launch_cte(p, dtype, static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------ gdn_cte_fused
namespace {
size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
struct FusedLayout {
  size_t qn, kn, g, beta, cte, total;  // byte offsets and total size
};
FusedLayout fused_layout(int B, int Hk, int Hv, int S, int Dk, int dtype) {
  FusedLayout L{};
  const size_t nqk = align256((size_t)B * Hk * S * Dk * esize(dtype));
  const size_t ng = align256((size_t)B * Hv * S * 4);
  L.qn = 0;
  L.kn = L.qn + nqk;
  L.g = L.kn + nqk;
  L.beta = L.g + ng;
  L.cte = L.beta + ng;
  L.total = L.cte + gdn::cte_workspace_bytes(B, Hv, S, dtype);
  return L;
}
}  // namespace

size_t gdn_cte_fused_workspace_size(int B, int Hk, int Hv, int S, int Dk, int Dv, int dtype) {
  (void)Dv;
  if (B <= 0 || Hk <= 0 || Hv <= 0 || S <= 0 || Dk <= 0 || (dtype != GDN_F32 && dtype != GDN_BF16)) return 0;
  return fused_layout(B, Hk, Hv, S, Dk, dtype).total;
}

int gdn_cte_fused(const void* q, const void* k, const void* v, const float* b, const float* a,
                  const float* A_log, const float* dt_bias, const void* z, const float* norm_weight,
                  float* recurrent_state, int has_initial_state, void* out, int B, int Hk, int Hv, int S,
                  int Dk, int Dv, int dtype, int algorithm, float rms_eps, void* workspace,
                  size_t workspace_bytes, void* stream) {
  if (dtype != GDN_F32 && dtype != GDN_BF16) return fail(GDN_ERR_DTYPE, "dtype %d is not GDN_F32 or GDN_BF16", dtype);
  if (algorithm != GDN_CTE_ALGO_DEFAULT && algorithm != GDN_CTE_ALGO_NEUMANN)
    return fail(GDN_ERR_UNSUPPORTED, "algorithm %d is not implemented (GDN_CTE_ALGO_DEFAULT or GDN_CTE_ALGO_NEUMANN)",
                algorithm);
  if (B < 0 || S < 0) return fail(GDN_ERR_SHAPE, "B=%d and S=%d must be >= 0", B, S);
  if (Hk < 1 || Hv < 1 || Hv % Hk != 0) return fail(GDN_ERR_SHAPE, "Hv=%d must be a positive multiple of Hk=%d", Hv, Hk);
  if (!head_dim_ok(Dk) || !head_dim_ok(Dv))
    return fail(GDN_ERR_SHAPE, "Dk=%d, Dv=%d must be multiples of 8 in [8, %d]", Dk, Dv, GDN_MAX_HEAD_DIM);
  if (!(rms_eps >= 0.f)) return fail(GDN_ERR_SHAPE, "rms_eps must be >= 0");
  if ((long long)B * Hv * ((Dv + 15) / 16) > 0x7fffffffLL) return fail(GDN_ERR_SHAPE, "B*Hv too large");
  const size_t es = esize(dtype);
  if ((size_t)S * 256 * es >= ((size_t)1 << 31))
    return fail(GDN_ERR_SHAPE, "S=%d is too long for one call (per-head data must stay below 2 GiB)", S);
  const size_t nqk = (size_t)B * Hk * S * Dk * es, nv = (size_t)B * Hv * S * Dv * es;
  const size_t ng = (size_t)B * Hv * S * 4, ns = (size_t)B * Hv * Dk * Dv * 4, nh = (size_t)Hv * 4;
  const Span sq{"q", q, nqk}, sk{"k", k, nqk}, sv{"v", v, nv}, sb{"b", b, ng}, sa{"a", a, ng},
      sal{"A_log", A_log, nh}, sdt{"dt_bias", dt_bias, nh}, sz{"z", z, nv},
      sw{"norm_weight", norm_weight, (size_t)Dv * 4}, st{"recurrent_state", recurrent_state, ns},
      so{"out", out, nv};
  if (int r = check_ptrs({sq, sk, sv, sb, sa, sal, sdt, sz, sw, st, so})) return r;
  if (int r = check_disjoint(so, {sq, sk, sv, sb, sa, sal, sdt, sz, sw, st})) return r;
  if (int r = check_disjoint(st, {sq, sk, sv, sb, sa, sal, sdt, sz, sw})) return r;
  if ((size_t)B * Hv == 0) return ok();
  const FusedLayout L = fused_layout(B, Hk, Hv, S, Dk, dtype);
  if (S > 0) {
    if (!workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL (%zu bytes required)", L.total);
    if (workspace_bytes < L.total)
      return fail(GDN_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", workspace_bytes, L.total);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(GDN_ERR_ALIGN, "workspace is not 256-byte aligned");
    const Span ws{"workspace", workspace, L.total};
    if (int r = check_disjoint(ws, {sq, sk, sv, sb, sa, sal, sdt, sz, sw, st, so})) return r;
  }
  if (int r = check_device()) return r;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(workspace);
  gdn::FusedPre f{};
  f.q = q; f.k = k;
  f.qn = S > 0 ? w + L.qn : nullptr;
  f.kn = S > 0 ? w + L.kn : nullptr;
  f.b = b; f.a = a; f.A_log = A_log; f.dt_bias = dt_bias;
  f.g = S > 0 ? reinterpret_cast<float*>(w + L.g) : nullptr;
  f.beta = S > 0 ? reinterpret_cast<float*>(w + L.beta) : nullptr;
  f.rows_qk = (long)B * Hk * S;
  f.tokens_v = (long)B * Hv * S;
  f.S = S; f.Hv = Hv; f.Dk = Dk;
  gdn::CteParams p{};
  hipError_t e = hipSuccess;
  if (dtype == GDN_BF16) {
    // bf16: the chunk-local kernel forms the unit rows and the gates itself
    // (into the same workspace areas), so no separate passes run
    p.q_raw = q; p.k_raw = k; p.b_raw = b; p.a_raw = a; p.A_log = A_log; p.dt_bias = dt_bias;
    p.qn = f.qn; p.kn = f.kn; p.g_out = f.g; p.beta_out = f.beta;
  } else if ((e = gdn::launch_fused_pre(f, dtype, hs)) != hipSuccess) {
    return launched(e);
  }
  p.q = f.qn; p.k = f.kn; p.v = v; p.g = f.g; p.beta = f.beta;
  p.state = recurrent_state; p.out = out;
  p.B = B; p.Hk = Hk; p.Hv = Hv; p.S = S; p.Dk = Dk; p.Dv = Dv;
  p.has_initial_state = has_initial_state ? 1 : 0;
  p.scale = 1.0f / sqrtf((float)Dk);
  p.algo = algorithm;
  p.ws = S > 0 ? w + L.cte : nullptr;
  e = gdn::launch_cte(p, dtype, hs);
  if (e != hipSuccess) return launched(e);
  gdn::FusedPost post{};
  post.out = out; post.z = z; post.norm_weight = norm_weight;
  post.rows = (long)B * Hv * S;
  post.Dv = Dv;
  post.rms_eps = rms_eps;
  return launched(gdn::launch_fused_post(post, dtype, hs));
}

// ------------------------------------------------------------ gdn_block_cte
namespace {
struct BlockCteLayout {
  size_t mixed, ztok, abtok, q, k, v, a, b, g, beta, o, cte, total;  // byte offsets and total size
};
BlockCteLayout block_cte_layout(int B, int S, int Hk, int Hv, int Dk, int Dv) {
  BlockCteLayout L{};
  const size_t M = (size_t)B * S, key_dim = (size_t)Hk * Dk, value_dim = (size_t)Hv * Dv;
  const size_t conv_dim = 2 * key_dim + value_dim, nh = align256(M * Hv * 4);
  size_t off = 0;
  L.mixed = off; off += align256(M * conv_dim * 2);
  L.ztok = off; off += align256(M * value_dim * 2);
  L.abtok = off; off += align256(2 * M * Hv * 2);
  L.q = off; off += align256(M * key_dim * 2);
  L.k = off; off += align256(M * key_dim * 2);
  L.v = off; off += align256(M * value_dim * 2);
  L.a = off; off += nh;
  L.b = off; off += nh;
  L.g = off; off += nh;
  L.beta = off; off += nh;
  L.o = off; off += align256(M * value_dim * 2);
  L.cte = off;
  L.total = off + gdn::cte_workspace_bytes(B, Hv, S, GDN_BF16);
  return L;
}
}  // namespace

size_t gdn_block_cte_workspace_size(int B, int S, int H, int num_k_heads, int num_v_heads, int head_k_dim,
                                    int head_v_dim, int K_win) {
  (void)H;
  (void)K_win;
  if (B <= 0 || S <= 0 || num_k_heads <= 0 || num_v_heads <= 0 || head_k_dim <= 0 || head_v_dim <= 0) return 0;
  return block_cte_layout(B, S, num_k_heads, num_v_heads, head_k_dim, head_v_dim).total;
}

int gdn_block_cte(const void* hidden, const void* W_in_qkv, const void* W_in_z, const void* W_in_a,
                  const void* W_in_b, const float* conv_weight, const void* conv_state_in, const float* A_log,
                  const float* dt_bias, const float* norm_weight, const float* recurrent_state_in, void* out,
                  void* conv_state_out, float* recurrent_state_out, int B, int S, int H, int num_k_heads,
                  int num_v_heads, int head_k_dim, int head_v_dim, int K_win, int algorithm, float rms_eps,
                  void* workspace, size_t workspace_bytes, void* stream) {
  const int Hk = num_k_heads, Hv = num_v_heads, Dk = head_k_dim, Dv = head_v_dim;
  if (algorithm != GDN_CTE_ALGO_DEFAULT && algorithm != GDN_CTE_ALGO_NEUMANN)
    return fail(GDN_ERR_UNSUPPORTED, "algorithm %d is not implemented (GDN_CTE_ALGO_DEFAULT or GDN_CTE_ALGO_NEUMANN)",
                algorithm);
  if (B < 0 || S < 0) return fail(GDN_ERR_SHAPE, "B=%d and S=%d must be >= 0", B, S);
  if (H < 128 || H % 128 != 0) return fail(GDN_ERR_SHAPE, "H=%d must be a positive multiple of 128", H);
  if (Hk < 1 || Hv < 1 || Hv % Hk != 0)
    return fail(GDN_ERR_SHAPE, "num_v_heads=%d must be a positive multiple of num_k_heads=%d", Hv, Hk);
  if (!head_dim_ok(Dk) || !head_dim_ok(Dv))
    return fail(GDN_ERR_SHAPE, "head dims %d, %d must be multiples of 8 in [8, %d]", Dk, Dv, GDN_MAX_HEAD_DIM);
  if (K_win < 1 || K_win > 8) return fail(GDN_ERR_SHAPE, "K_win=%d must be in [1, 8]", K_win);
  if (!(rms_eps >= 0.f)) return fail(GDN_ERR_SHAPE, "rms_eps must be >= 0");
  const size_t M = (size_t)B * S, key_dim = (size_t)Hk * Dk, value_dim = (size_t)Hv * Dv;
  const size_t conv_dim = 2 * key_dim + value_dim;
  const size_t lim = (size_t)1 << 31;
  if (M * H * 2 >= lim || (size_t)H * conv_dim * 2 >= lim || M * conv_dim * 2 >= lim || M * value_dim * 2 >= lim ||
      (size_t)B * conv_dim * K_win * 2 >= lim || (size_t)S * 256 * 2 >= lim)
    return fail(GDN_ERR_SHAPE, "a buffer reaches 2 GiB (B=%d, S=%d, H=%d)", B, S, H);
  const size_t ns = (size_t)B * Hv * Dk * Dv * 4, ncs = (size_t)B * conv_dim * K_win * 2;
  const Span sh{"hidden", hidden, M * H * 2}, swq{"W_in_qkv", W_in_qkv, (size_t)H * conv_dim * 2},
      swz{"W_in_z", W_in_z, (size_t)H * value_dim * 2}, swa{"W_in_a", W_in_a, (size_t)H * Hv * 2},
      swb{"W_in_b", W_in_b, (size_t)H * Hv * 2}, scw{"conv_weight", conv_weight, conv_dim * K_win * 4},
      scs{"conv_state_in", conv_state_in, ncs}, sal{"A_log", A_log, (size_t)Hv * 4},
      sdt{"dt_bias", dt_bias, (size_t)Hv * 4}, snw{"norm_weight", norm_weight, (size_t)Dv * 4},
      srs{"recurrent_state_in", recurrent_state_in, ns}, so{"out", out, M * value_dim * 2},
      sco{"conv_state_out", conv_state_out, ncs}, sro{"recurrent_state_out", recurrent_state_out, ns};
  if (int r = check_ptrs({sh, swq, swz, swa, swb, scw, scs, sal, sdt, snw, srs, so, sco, sro})) return r;
  const std::vector<Span> ins{sh, swq, swz, swa, swb, scw, scs, sal, sdt, snw, srs};
  if (int r = check_disjoint(so, {sh, swq, swz, swa, swb, scw, scs, sal, sdt, snw, srs, sco, sro})) return r;
  if (int r = check_disjoint(sco, ins, conv_state_in)) return r;
  if (int r = check_disjoint(sro, ins, recurrent_state_in)) return r;
  if (int r = check_disjoint(sco, {sro})) return r;
  if (B == 0) return ok();
  const BlockCteLayout L = block_cte_layout(B, S, Hk, Hv, Dk, Dv);
  if (S > 0) {
    if (!workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL (%zu bytes required)", L.total);
    if (workspace_bytes < L.total)
      return fail(GDN_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", workspace_bytes, L.total);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(GDN_ERR_ALIGN, "workspace is not 256-byte aligned");
    const Span ws{"workspace", workspace, L.total};
    if (int r = check_disjoint(ws, {sh, swq, swz, swa, swb, scw, scs, sal, sdt, snw, srs, so, sco, sro})) return r;
  }
  if (int r = check_device()) return r;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (recurrent_state_out != recurrent_state_in)
    e = hipMemcpyAsync(recurrent_state_out, recurrent_state_in, ns, hipMemcpyDeviceToDevice, hs);
  if (e != hipSuccess) return launched(e);
  if (S == 0) {
    if (conv_state_out != conv_state_in)
      e = hipMemcpyAsync(conv_state_out, conv_state_in, ncs, hipMemcpyDeviceToDevice, hs);
    return launched(e);
  }
  char* w = static_cast<char*>(workspace);
  // The q|k|v and z projections are plain GEMMs and go to the vendor
  // library; what it does not take runs in one launch of gemm_bf16_kernel.
  // The narrow a and b projections (N = Hv) run as one MFMA kernel that
  // reads hidden once and writes them head-major (Hv a multiple of 16 up to
  // 64); other Hv join the GEMMs when their rows are whole 16-byte pieces,
  // else they take one wave per token.
  const bool ab_mfma = Hv % 16 == 0 && Hv <= 64;
  const bool ab_gemm = !ab_mfma && Hv % 8 == 0;
  gdn::GemmParams gp{};
  gp.A = hidden; gp.M = (int)M; gp.K = H;
  auto add = [&](const void* Wm, void* Cm, int N) {
    gp.B[gp.nprob] = Wm; gp.C[gp.nprob] = Cm; gp.N[gp.nprob] = N;
    ++gp.nprob;
  };
  if (gdn::gemm_bf16_library(hidden, W_in_qkv, w + L.mixed, (int)M, (int)conv_dim, H, hs) != hipSuccess)
    add(W_in_qkv, w + L.mixed, (int)conv_dim);
  if (gdn::gemm_bf16_library(hidden, W_in_z, w + L.ztok, (int)M, (int)value_dim, H, hs) != hipSuccess)
    add(W_in_z, w + L.ztok, (int)value_dim);
  if (ab_gemm) {
    if (gdn::gemm_bf16_library(hidden, W_in_a, w + L.abtok, (int)M, Hv, H, hs) != hipSuccess)
      add(W_in_a, w + L.abtok, Hv);
    if (gdn::gemm_bf16_library(hidden, W_in_b, w + L.abtok + M * Hv * 2, (int)M, Hv, H, hs) != hipSuccess)
      add(W_in_b, w + L.abtok + M * Hv * 2, Hv);
  }
  if (gp.nprob > 0 && (e = gdn::launch_gemm_bf16(gp, hs)) != hipSuccess) return launched(e);
  if (!ab_gemm) {
    gdn::NarrowParams na{hidden, W_in_a, W_in_b, reinterpret_cast<float*>(w + L.a),
                         reinterpret_cast<float*>(w + L.b), (int)M, Hv, H, S};
    if ((e = ab_mfma ? gdn::launch_proj_ab(na, hs) : gdn::launch_proj_narrow(na, hs)) != hipSuccess)
      return launched(e);
  }
  gdn::ConvSplitParams cs{};
  cs.ab_tok = ab_gemm ? w + L.abtok : nullptr;
  cs.a_head = reinterpret_cast<float*>(w + L.a);
  cs.b_head = reinterpret_cast<float*>(w + L.b);
  // (z stays token-major: the output norm reads it there)
  cs.mixed = w + L.mixed; cs.conv_weight = conv_weight; cs.conv_state = conv_state_in;
  cs.conv_state_out = conv_state_out; cs.q = w + L.q; cs.k = w + L.k; cs.v = w + L.v;
  cs.B = B; cs.S = S; cs.conv_dim = (int)conv_dim; cs.value_dim = (int)value_dim; cs.key_dim = (int)key_dim;
  cs.Hk = Hk; cs.Hv = Hv; cs.Dk = Dk; cs.Dv = Dv; cs.K_win = K_win;
  if ((e = gdn::launch_conv_split(cs, hs)) != hipSuccess) return launched(e);
  gdn::FusedPre f{};
  f.q = w + L.q; f.k = w + L.k; f.qn = w + L.q; f.kn = w + L.k;
  f.b = reinterpret_cast<float*>(w + L.b); f.a = reinterpret_cast<float*>(w + L.a);
  f.A_log = A_log; f.dt_bias = dt_bias;
  f.g = reinterpret_cast<float*>(w + L.g); f.beta = reinterpret_cast<float*>(w + L.beta);
  f.rows_qk = (long)B * Hk * S; f.tokens_v = (long)B * Hv * S;
  f.S = S; f.Hv = Hv; f.Dk = Dk;
  gdn::CteParams p{};
  if (gdn::fused_inplace_ok(Hk, Hv)) {
    // the chunk-local kernel forms the unit rows over the raw ones (one
    // workgroup reads and writes each key head's chunk) and the gates
    p.q_raw = f.q; p.k_raw = f.k; p.b_raw = f.b; p.a_raw = f.a; p.A_log = A_log; p.dt_bias = dt_bias;
    p.qn = f.qn; p.kn = f.kn; p.g_out = f.g; p.beta_out = f.beta;
  } else if ((e = gdn::launch_fused_pre(f, GDN_BF16, hs)) != hipSuccess) {
    return launched(e);
  }
  p.q = w + L.q; p.k = w + L.k; p.v = w + L.v; p.g = f.g; p.beta = f.beta;
  p.state = recurrent_state_out; p.out = w + L.o;
  p.B = B; p.Hk = Hk; p.Hv = Hv; p.S = S; p.Dk = Dk; p.Dv = Dv;
  p.has_initial_state = 1;
  p.scale = 1.0f / sqrtf((float)Dk);
  p.algo = algorithm;
  p.ws = w + L.cte;
  if ((e = gdn::launch_cte(p, GDN_BF16, hs)) != hipSuccess) return launched(e);
  gdn::FusedPost post{};
  post.out = w + L.o; post.z = w + L.ztok; post.norm_weight = norm_weight;
  post.rows = (long)B * Hv * S; post.Dv = Dv; post.rms_eps = rms_eps;
  post.out_tok = out; post.S = S; post.Hv = Hv; post.z_token_major = 1;
  return launched(gdn::launch_fused_post(post, GDN_BF16, hs));
}

// ------------------------------------------------------------------ gdn_tkg
int gdn_tkg(const void* q, const void* k, const void* v, const float* b, const float* a,
            const float* A_log, const float* dt_bias, const void* z, const float* norm_weight,
            const float* state_in, float* state_out, void* out, int BH, int num_v_heads, int K, int V,
            int dtype, float rms_eps, void* stream) {
  if (dtype != GDN_F32 && dtype != GDN_BF16) return fail(GDN_ERR_DTYPE, "dtype %d is not GDN_F32 or GDN_BF16", dtype);
  if (BH < 0 || num_v_heads < 1 || BH % num_v_heads != 0)
    return fail(GDN_ERR_SHAPE, "BH=%d must be a non-negative multiple of num_v_heads=%d", BH, num_v_heads);
  if (!head_dim_ok(K) || !head_dim_ok(V))
    return fail(GDN_ERR_SHAPE, "K=%d, V=%d must be multiples of 8 in [8, %d]", K, V, GDN_MAX_HEAD_DIM);
  if (!(rms_eps >= 0.f)) return fail(GDN_ERR_SHAPE, "rms_eps must be >= 0");
  const size_t es = esize(dtype);
  const Span sq{"q", q, (size_t)BH * K * es}, sk{"k", k, (size_t)BH * K * es}, sv{"v", v, (size_t)BH * V * es},
      sz{"z", z, (size_t)BH * V * es}, sb{"b", b, (size_t)BH * 4}, sa{"a", a, (size_t)BH * 4},
      sal{"A_log", A_log, (size_t)num_v_heads * 4}, sdt{"dt_bias", dt_bias, (size_t)num_v_heads * 4},
      sw{"norm_weight", norm_weight, (size_t)V * 4}, si{"state_in", state_in, (size_t)BH * K * V * 4},
      so{"state_out", state_out, (size_t)BH * K * V * 4}, sy{"out", out, (size_t)BH * V * 2};
  if (BH == 0) return ok();
  if (int r = check_ptrs({sq, sk, sv, sz, sb, sa, sal, sdt, sw, si, so, sy})) return r;
  if (int r = check_disjoint(so, {sq, sk, sv, sz, sb, sa, sal, sdt, sw, si}, state_in)) return r;
  if (int r = check_disjoint(sy, {sq, sk, sv, sz, sb, sa, sal, sdt, sw, si, so})) return r;
  if (int r = check_device()) return r;
  gdn::TkgParams p;
  p.q = q; p.k = k; p.qk_bstride = (long)num_v_heads * K; p.head_div = 1;
  p.v = v; p.v_bstride = (long)num_v_heads * V; p.z = z;
  p.b = b; p.a = a; p.A_log = A_log; p.dt_bias = dt_bias; p.norm_weight = norm_weight;
  p.state_in = state_in; p.state_out = state_out; p.out = out;
  p.BH = BH; p.Hv = num_v_heads; p.K = K; p.V = V; p.rms_eps = rms_eps;
  return launched(gdn::launch_tkg(p, dtype, static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------ gdn_block_tkg
size_t gdn_block_tkg_workspace_size(int B, int H, int num_k_heads, int num_v_heads, int head_k_dim,
                                    int head_v_dim, int K_win) {
  (void)H;
  (void)K_win;
  if (B <= 0 || num_k_heads <= 0 || num_v_heads <= 0 || head_k_dim <= 0 || head_v_dim <= 0) return 0;
  return gdn::block_workspace_layout(B, num_k_heads, num_v_heads, head_k_dim, head_v_dim).total;
}

int gdn_block_tkg(const void* hidden, const void* W_in_qkv, const void* W_in_z, const void* W_in_a,
                  const void* W_in_b, const float* conv_weight, const void* conv_state_in,
                  const float* A_log, const float* dt_bias, const float* norm_weight,
                  const float* recurrent_state_in, void* out, void* conv_state_out,
                  float* recurrent_state_out, int B, int H, int num_k_heads, int num_v_heads,
                  int head_k_dim, int head_v_dim, int K_win, float rms_eps, void* workspace,
                  size_t workspace_bytes, void* stream) {
  const int Hk = num_k_heads, Hv = num_v_heads, Dk = head_k_dim, Dv = head_v_dim;
  if (B < 0) return fail(GDN_ERR_SHAPE, "B=%d must be >= 0", B);
  if (H < 128 || H % 128 != 0) return fail(GDN_ERR_SHAPE, "H=%d must be a positive multiple of 128", H);
  if (Hk < 1 || Hv < 1 || Hv % Hk != 0)
    return fail(GDN_ERR_SHAPE, "num_v_heads=%d must be a positive multiple of num_k_heads=%d", Hv, Hk);
  if (!head_dim_ok(Dk) || !head_dim_ok(Dv))
    return fail(GDN_ERR_SHAPE, "head dims %d, %d must be multiples of 8 in [8, %d]", Dk, Dv, GDN_MAX_HEAD_DIM);
  if (K_win < 1 || K_win > 8) return fail(GDN_ERR_SHAPE, "K_win=%d must be in [1, 8]", K_win);
  if (!(rms_eps >= 0.f)) return fail(GDN_ERR_SHAPE, "rms_eps must be >= 0");
  if (B == 0) return ok();
  const size_t key_dim = (size_t)Hk * Dk, value_dim = (size_t)Hv * Dv;
  const size_t conv_dim = 2 * key_dim + value_dim;
  // weights and the hidden batch are addressed with 32-bit buffer offsets below 2^31
  if ((size_t)H * conv_dim * 2 >= ((size_t)1 << 31) || (size_t)B * H * 2 >= ((size_t)1 << 31) ||
      (size_t)B * conv_dim * K_win * 2 >= ((size_t)1 << 31))
    return fail(GDN_ERR_SHAPE, "H=%d x conv_dim=%zu weights (or the hidden batch, or the conv state) exceed 2 GiB",
                H, conv_dim);
  const Span sh{"hidden", hidden, (size_t)B * H * 2}, swq{"W_in_qkv", W_in_qkv, (size_t)H * conv_dim * 2},
      swz{"W_in_z", W_in_z, (size_t)H * value_dim * 2}, swa{"W_in_a", W_in_a, (size_t)H * Hv * 2},
      swb{"W_in_b", W_in_b, (size_t)H * Hv * 2}, scw{"conv_weight", conv_weight, conv_dim * K_win * 4},
      sci{"conv_state_in", conv_state_in, (size_t)B * conv_dim * K_win * 2},
      sal{"A_log", A_log, (size_t)Hv * 4}, sdt{"dt_bias", dt_bias, (size_t)Hv * 4},
      snw{"norm_weight", norm_weight, (size_t)Dv * 4},
      sri{"recurrent_state_in", recurrent_state_in, (size_t)B * Hv * Dk * Dv * 4},
      sy{"out", out, (size_t)B * value_dim * 2},
      sco{"conv_state_out", conv_state_out, (size_t)B * conv_dim * K_win * 2},
      sro{"recurrent_state_out", recurrent_state_out, (size_t)B * Hv * Dk * Dv * 4};
  const gdn::BlockWorkspace L = gdn::block_workspace_layout(B, Hk, Hv, Dk, Dv);
  const Span sws{"workspace", workspace, L.total};
  if (int r = check_ptrs({sh, swq, swz, swa, swb, scw, sci, sal, sdt, snw, sri, sy, sco, sro})) return r;
  if (!workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL (%zu bytes required)", L.total);
  if (workspace_bytes < L.total)
    return fail(GDN_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", workspace_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(GDN_ERR_ALIGN, "workspace is not 256-byte aligned");
  const std::vector<Span> ins = {sh, swq, swz, swa, swb, scw, sci, sal, sdt, snw, sri};
  if (int r = check_disjoint(sy, ins)) return r;
  if (int r = check_disjoint(sco, ins, conv_state_in)) return r;
  if (int r = check_disjoint(sro, ins, recurrent_state_in)) return r;
  if (int r = check_disjoint(sws, ins)) return r;
  if (int r = check_disjoint(sy, {sco, sro, sws})) return r;
  if (int r = check_disjoint(sco, {sro, sws})) return r;
  if (int r = check_disjoint(sro, {sws})) return r;
  if (int r = check_device()) return r;

  char* ws = static_cast<char*>(workspace);
  gdn::BlockParams bp;
  bp.hidden = hidden; bp.W_qkv = W_in_qkv; bp.W_z = W_in_z; bp.W_a = W_in_a; bp.W_b = W_in_b;
  bp.conv_weight = conv_weight; bp.conv_state_in = conv_state_in; bp.conv_state_out = conv_state_out;
  bp.ws_conv_out = ws + L.conv_out; bp.ws_z = ws + L.z;
  bp.ws_a = reinterpret_cast<float*>(ws + L.a); bp.ws_b = reinterpret_cast<float*>(ws + L.b);
  bp.B = B; bp.H = H; bp.Hk = Hk; bp.Hv = Hv; bp.Dk = Dk; bp.Dv = Dv; bp.K_win = K_win;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = gdn::launch_block_proj(bp, st);
  if (e != hipSuccess) return launched(e);

  const uint16_t* act = static_cast<const uint16_t*>(bp.ws_conv_out);  // bf16 elements
  gdn::TkgParams p;
  p.q = act;
  p.k = act + key_dim;
  p.qk_bstride = (long)conv_dim;
  p.head_div = Hv / Hk;
  p.v = act + 2 * key_dim;
  p.v_bstride = (long)conv_dim;
  p.z = bp.ws_z;
  p.b = bp.ws_b; p.a = bp.ws_a; p.A_log = A_log; p.dt_bias = dt_bias; p.norm_weight = norm_weight;
  p.state_in = recurrent_state_in; p.state_out = recurrent_state_out; p.out = out;
  p.BH = B * Hv; p.Hv = Hv; p.K = Dk; p.V = Dv; p.rms_eps = rms_eps;
  return launched(gdn::launch_tkg(p, GDN_BF16, st));
}

}  // extern "C"
