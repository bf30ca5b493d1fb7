// extern "C" entry points of libstarkv: argument checks, then launches on the caller's stream.
#include <math.h>
#include <stdint.h>

#include <string.h>

#include <cmath>
#include <mutex>
#include <new>
#include <vector>

#include "device_common.h"
#include "profile.h"
#include "starkv_internal.h"

namespace skv {
int layer_init(const starkv_layer_desc& d, Layer* L);
int layer_upload_tables(Layer* L);
int layer_write_rope(Layer* L);
}  // namespace skv

// The last decode plan of a layer, reused while the batch, query count and lengths repeat (a
// decode loop calls workspace_bytes and then the decode with the same lengths; a serving loop
// repeats them while the lengths do not change).  The plan depends on the cache capacity and the
// workspace address only through the capacity field and the workspace pointers, which a hit
// rebases.
struct PlanMemo {
  std::mutex mu;
  bool valid = false;
  int B = 0, n_q = 0;
  std::vector<int32_t> lens;
  uintptr_t ws_base = 0;
  skv::DecodePlan plan;
  skv::KtList kts;
  skv::SeqTable seq;
};

struct starkv_layer {
  skv::Layer L;
  PlanMemo memo;
};

// Device scratch of starkv_decode_step_noalloc: one array per GPU, in the library's code object,
// held until the process ends.  Host code never uses the array's name as an address (on the host
// it only names the symbol): the device address of each GPU's copy is looked up once per device
// with hipGetSymbolAddress, and that pointer is what the kernels receive.
constexpr size_t kScratchBytes = (size_t)STARKV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of the scratch array (looked up on the first call on that device).
static int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return STARKV_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return STARKV_EUNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return STARKV_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return STARKV_OK;
}

static void rebase_plan(skv::DecodePlan* P, uintptr_t from, uintptr_t to, int T_max) {
  auto rb = [&](auto*& p) { p = reinterpret_cast<std::remove_reference_t<decltype(p)>>((uintptr_t)p - from + to); };
  skv::DecodeWs& w = P->ws;
  rb(w.qfrag);
  rb(w.rowp);
  rb(w.p);
  rb(w.cm);
  rb(w.cl);
  rb(w.zp);
  rb(w.sl);
  rb(w.sm);
  rb(w.zt);
  rb(w.qraw);
  P->g.T_max = T_max;
}

// plan_decode through the layer's memo (thread-safe: the memo has its own lock)
static int get_plan(const starkv_layer* l, int B, int n_q, const int32_t* lens, int T_max, void* ws,
                    skv::DecodePlan* plan, skv::KtList* kts, skv::SeqTable* seq) {
  PlanMemo& m = const_cast<PlanMemo&>(l->memo);
  std::lock_guard<std::mutex> lk(m.mu);
  if (m.valid && m.B == B && m.n_q == n_q && memcmp(m.lens.data(), lens, sizeof(int32_t) * B) == 0) {
    *plan = m.plan;
    *kts = m.kts;
    *seq = m.seq;
    rebase_plan(plan, m.ws_base, (uintptr_t)ws, T_max);
    return STARKV_OK;
  }
  const int st = skv::plan_decode(l->L, B, n_q, lens, T_max, ws, plan, kts, seq);
  if (st != STARKV_OK) return st;
  m.valid = true;
  m.B = B;
  m.n_q = n_q;
  m.lens.assign(lens, lens + B);
  m.ws_base = (uintptr_t)ws;
  m.plan = *plan;
  m.kts = *kts;
  m.seq = *seq;
  return STARKV_OK;
}

using skv::Layer;

#define SKV_GUARD_BEGIN try {
#define SKV_GUARD_END                 \
  }                                   \
  catch (const std::bad_alloc&) {     \
    return STARKV_ENOMEM;             \
  }                                   \
  catch (...) {                       \
    return STARKV_EINVAL;             \
  }

static int hip_status(hipError_t e) { return e == hipSuccess ? STARKV_OK : STARKV_EHIP; }

static bool bad_float(float x) { return !(x == x) || isinf(x); }

// The layer's small device tables are allocated by the first setup call that binds factors.
static int ensure_tables(Layer* L) {
  if (L->dev_tables) return STARKV_OK;
  return skv::layer_upload_tables(L);
}

extern "C" {

int starkv_abi_version(void) { return STARKV_ABI_VERSION; }

const char* starkv_status_string(int status) {
  switch (status) {
    case STARKV_OK: return "ok";
    case STARKV_EINVAL: return "invalid argument";
    case STARKV_ENOMEM: return "out of memory";
    case STARKV_ECAPACITY: return "cache capacity exceeded";
    case STARKV_EUNSUPPORTED: return "unsupported configuration";
    case STARKV_EWORKSPACE: return "workspace too small";
    case STARKV_EHIP: return "HIP runtime error";
    case STARKV_ESTATE: return "factors or scales not bound";
    default: return "unknown status";
  }
}

int starkv_layer_create(const starkv_layer_desc* d, starkv_layer** out) {
  SKV_GUARD_BEGIN
  if (!d || !out) return STARKV_EINVAL;
  *out = nullptr;
  if (d->H_q <= 0 || d->H_kv <= 0 || d->d_h <= 0 || d->d <= 0 || d->n_v <= 0) return STARKV_EINVAL;
  if (d->H_q % d->H_kv != 0) return STARKV_EINVAL;
  if (!d->s_k || !d->tau_k || !d->s_v) return STARKV_EINVAL;
  if (d->dtype != STARKV_F32 && d->dtype != STARKV_BF16) return STARKV_EINVAL;
  if (d->latent != STARKV_LATENT_F32 && d->latent != STARKV_LATENT_BF16 && d->latent != STARKV_LATENT_MIX84 &&
      d->latent != STARKV_LATENT_HAD43 && d->latent != STARKV_LATENT_HAD43P)
    return STARKV_EINVAL;
  if (d->shrink != 0 && d->shrink != 1) return STARKV_EINVAL;
  if (bad_float(d->tau_v) || d->tau_v < 0.f) return STARKV_EINVAL;
  for (int g = 0; g < d->H_kv; ++g)
    if (bad_float(d->tau_k[g]) || d->tau_k[g] < 0.f) return STARKV_EINVAL;
  for (long i = 0; i < (long)d->H_kv * d->d_h; ++i)
    if (bad_float(d->s_k[i])) return STARKV_EINVAL;
  for (int i = 0; i < d->n_v; ++i)
    if (bad_float(d->s_v[i])) return STARKV_EINVAL;
  // the rank is the count of values above the threshold, taken as a prefix: the spectra must be
  // descending (ties allowed), as singular values are
  for (int g = 0; g < d->H_kv; ++g)
    for (int i = 1; i < d->d_h; ++i)
      if (d->s_k[(long)g * d->d_h + i] > d->s_k[(long)g * d->d_h + i - 1]) return STARKV_EINVAL;
  for (int i = 1; i < d->n_v; ++i)
    if (d->s_v[i] > d->s_v[i - 1]) return STARKV_EINVAL;
  // supported combinations and sizes
  if (d->latent == STARKV_LATENT_F32 && d->dtype != STARKV_F32) return STARKV_EUNSUPPORTED;
  if (d->latent != STARKV_LATENT_F32 && d->dtype != STARKV_BF16) return STARKV_EUNSUPPORTED;
  if (d->d % 16 != 0 || d->d_h % 32 != 0 || d->d_h > 256) return STARKV_EUNSUPPORTED;
  if (d->latent == STARKV_LATENT_HAD43P && d->d % 64 != 0) return STARKV_EUNSUPPORTED;
  if (d->n_v > d->d || d->n_v > d->H_kv * d->d_h) return STARKV_EINVAL;
  starkv_layer* l = new starkv_layer();
  int st = skv::layer_init(*d, &l->L);
  if (st == STARKV_OK && (l->L.n_lat > 8192 || l->L.H_kv * l->L.d_h > 65536)) st = STARKV_EUNSUPPORTED;
  if (st != STARKV_OK) {
    delete l;
    return st;
  }
  *out = l;
  return STARKV_OK;
  SKV_GUARD_END
}

int starkv_layer_destroy(starkv_layer* l) {
  if (!l) return STARKV_EINVAL;
  if (l->L.dev_tables) (void)hipFree(l->L.dev_tables);
  if (l->L.d_wqk) (void)hipFree(l->L.d_wqk);
  delete l;
  return STARKV_OK;
}

int starkv_layer_get_info(const starkv_layer* l, starkv_layer_info* info) {
  if (!l || !info) return STARKV_EINVAL;
  const Layer& L = l->L;
  info->H_q = L.H_q;
  info->H_kv = L.H_kv;
  info->d_h = L.d_h;
  info->d = L.d;
  info->dtype = L.dtype;
  info->latent = L.pack3 ? STARKV_LATENT_HAD43P : (L.had ? STARKV_LATENT_HAD43 : L.latent);
  info->n_key = L.n_key;
  info->r_v = L.r_v;
  info->n_lat = L.n_lat;
  info->k_row_bytes = L.k_row_bytes;
  info->v_tile_rows = L.v_rows;
  info->v_tile_bytes = L.v_tile_bytes;
  info->K8 = L.K8;
  info->K4 = L.K4;
  info->V8 = L.V8;
  info->V4 = L.V4;
  info->K3 = L.K3;
  info->V3 = L.V3;
  const size_t es = L.dtype == STARKV_F32 ? 4 : 2;
  info->a_bytes = (size_t)L.n_lat * L.d * es;
  info->bk_bytes = (size_t)L.n_key * L.d_h * es;
  info->bv_bytes = (size_t)L.H_kv * L.d_h * L.r_v * es;
  info->scale_bytes = L.mix() ? (size_t)L.n_lat * 2 : 0;
  return STARKV_OK;
}

int starkv_layer_ranks(const starkv_layer* l, int32_t* ranks_out) {
  if (!l || !ranks_out) return STARKV_EINVAL;
  for (int g = 0; g < l->L.H_kv; ++g) ranks_out[g] = l->L.rk[g];
  ranks_out[l->L.H_kv] = l->L.r_v;
  return STARKV_OK;
}

// absorbed query factors depend on the bound B_k: binding new factors drops them
static void drop_absorbed(Layer* L) {
  if (L->d_wqk) (void)hipFree(L->d_wqk);
  L->d_wqk = nullptr;
}

int starkv_build_factors(starkv_layer* l, const float* U_k, const float* V_k, const float* U_v, const float* V_v,
                         void* A_t, void* B_k, void* B_vt, hipStream_t stream) {
  SKV_GUARD_BEGIN
  if (!l || !U_k || !V_k || !U_v || !V_v || !A_t || !B_k || !B_vt) return STARKV_EINVAL;
  int st = ensure_tables(&l->L);
  if (st != STARKV_OK) return st;
  st = hip_status(skv::launch_build_factors(l->L, U_k, V_k, U_v, V_v, A_t, B_k, B_vt, stream));
  if (st == STARKV_OK) {
    l->L.A_t = A_t;
    l->L.B_k = B_k;
    l->L.B_vt = B_vt;
    drop_absorbed(&l->L);
  }
  return st;
  SKV_GUARD_END
}

int starkv_bind_factors(starkv_layer* l, const void* A_t, const void* B_k, const void* B_vt) {
  SKV_GUARD_BEGIN
  if (!l || !A_t || !B_k || !B_vt) return STARKV_EINVAL;
  int st = ensure_tables(&l->L);
  if (st != STARKV_OK) return st;
  l->L.A_t = A_t;
  l->L.B_k = B_k;
  l->L.B_vt = B_vt;
  drop_absorbed(&l->L);
  return STARKV_OK;
  SKV_GUARD_END
}

int starkv_absorb_query(starkv_layer* l, const void* W_q, hipStream_t stream) {
  SKV_GUARD_BEGIN
  if (!l || !W_q) return STARKV_EINVAL;
  Layer& L = l->L;
  if (!L.dev_tables || !L.B_k) return STARKV_ESTATE;
  if (!L.d_wqk) {
    const size_t bytes = (size_t)L.G * L.n_key * L.d * sizeof(float);
    if (hipMalloc((void**)&L.d_wqk, bytes) != hipSuccess) {
      L.d_wqk = nullptr;
      return STARKV_ENOMEM;
    }
  }
  const int st = hip_status(skv::launch_absorb_query(L, W_q, L.d_wqk, stream));
  if (st != STARKV_OK) drop_absorbed(&L);
  return st;
  SKV_GUARD_END
}

int starkv_calibrate(starkv_layer* l, const void* X_cal, int n_cal, uint16_t* scales_out, hipStream_t stream) {
  SKV_GUARD_BEGIN
  if (!l || !X_cal || !scales_out || n_cal <= 0) return STARKV_EINVAL;
  if (!l->L.mix()) return STARKV_EUNSUPPORTED;
  if (!l->L.A_t) return STARKV_ESTATE;
  int st = hip_status(skv::launch_calibrate(l->L, X_cal, n_cal, scales_out, stream));
  if (st == STARKV_OK) l->L.scales = scales_out;
  return st;
  SKV_GUARD_END
}

int starkv_bind_scales(starkv_layer* l, const uint16_t* scales) {
  if (!l || !scales) return STARKV_EINVAL;
  if (!l->L.mix()) return STARKV_EUNSUPPORTED;
  l->L.scales = scales;
  return STARKV_OK;
}

// one sequence's key rows must be addressable by 32-bit buffer offsets below the out-of-range
// offset the kernels use for masked loads
constexpr size_t kMaxSeqKeyBytes = 0xFFFFFF00u;

int starkv_cache_bytes(const starkv_layer* l, int B, int T_max, size_t* k_bytes, size_t* v_bytes) {
  if (!l || !k_bytes || !v_bytes || B <= 0 || T_max <= 0 || T_max % STARKV_TILE_TOKENS != 0) return STARKV_EINVAL;
  if ((size_t)T_max * l->L.k_row_bytes >= kMaxSeqKeyBytes) return STARKV_EUNSUPPORTED;
  *k_bytes = (size_t)B * T_max * l->L.k_row_bytes;
  *v_bytes = (size_t)B * (T_max / STARKV_TILE_TOKENS) * l->L.v_tile_bytes;
  return STARKV_OK;
}

static int check_cache(const Layer& L, const starkv_cache* c, int B) {
  if (!c || !c->k_rows || !c->v_tiles) return STARKV_EINVAL;
  if (c->T_max <= 0 || c->T_max % STARKV_TILE_TOKENS != 0 || c->B <= 0) return STARKV_EINVAL;
  if (B > c->B) return STARKV_EINVAL;
  // the kernels address one sequence's key rows with 32-bit buffer offsets
  if ((size_t)c->T_max * L.k_row_bytes >= kMaxSeqKeyBytes) return STARKV_EUNSUPPORTED;
  return STARKV_OK;
}

static int check_bound(const Layer& L, bool need_bk) {
  if (!L.dev_tables || !L.A_t || !L.B_vt || (need_bk && !L.B_k)) return STARKV_ESTATE;
  if (L.mix() && !L.scales) return STARKV_ESTATE;
  return STARKV_OK;
}

// Device lengths: 4-byte aligned when given.
static bool lens_dev_ok(const int32_t* lens_dev) { return ((uintptr_t)lens_dev & 3) == 0; }

// Rotary layers whose decode attends over reconstructed keys and values plan on host lengths only.
static bool recon_decode(const Layer& L, int n_q) { return L.rope_theta > 0.f && !skv::rope_latent_scores(L, n_q); }

int starkv_compress_append(const starkv_layer* l, const starkv_cache* c, const void* X_new, int B, int n_new,
                           const int32_t* lens_host, const int32_t* lens_dev, hipStream_t stream) {
  SKV_GUARD_BEGIN
  if (!l || !lens_host || !lens_dev_ok(lens_dev)) return STARKV_EINVAL;
  if (B <= 0 || B > STARKV_MAX_BATCH || n_new < 0) return B > STARKV_MAX_BATCH ? STARKV_EUNSUPPORTED : STARKV_EINVAL;
  int st = check_cache(l->L, c, B);
  if (st != STARKV_OK) return st;
  if (n_new == 0) return STARKV_OK;
  if (!X_new) return STARKV_EINVAL;
  if ((long)B * n_new > (1L << 30)) return STARKV_EUNSUPPORTED;
  for (int b = 0; b < B; ++b) {
    if (lens_host[b] < 0) return STARKV_EINVAL;
    if ((long)lens_host[b] + n_new > c->T_max) return STARKV_ECAPACITY;
  }
  st = check_bound(l->L, false);
  if (st != STARKV_OK) return st;
  return hip_status(skv::launch_append(l->L, *c, X_new, B, n_new, lens_host, stream, lens_dev, 0));
  SKV_GUARD_END
}

static int check_decode(const Layer& L, const starkv_cache* c, int B, int n_q, const int32_t* lens) {
  if (!lens) return STARKV_EINVAL;
  if (B <= 0 || n_q <= 0) return STARKV_EINVAL;
  if (B > STARKV_MAX_BATCH || L.H_q * n_q > STARKV_MAX_QROWS) return STARKV_EUNSUPPORTED;
  int st = check_cache(L, c, B);
  if (st != STARKV_OK) return st;
  for (int b = 0; b < B; ++b) {
    if (lens[b] < n_q) return STARKV_EINVAL;
    if (lens[b] > c->T_max) return STARKV_ECAPACITY;
  }
  return STARKV_OK;
}

int starkv_decode_workspace_bytes(const starkv_layer* l, int B, int n_q, const int32_t* lens_host, size_t* bytes) {
  SKV_GUARD_BEGIN
  if (!l || !bytes || !lens_host || B <= 0 || n_q <= 0) return STARKV_EINVAL;
  if (B > STARKV_MAX_BATCH || l->L.H_q * n_q > STARKV_MAX_QROWS) return STARKV_EUNSUPPORTED;
  for (int b = 0; b < B; ++b)
    if (lens_host[b] < n_q) return STARKV_EINVAL;
  if (l->L.rope_theta > 0.f && !skv::rope_latent_scores(l->L, n_q)) {
    // rotary layers with more than 32 query rows per KV head attend over reconstructed K and V
    *bytes = skv::prefill_workspace_bytes(l->L, B, lens_host);
    return STARKV_OK;
  }
  skv::DecodePlan plan;
  skv::KtList kts;
  skv::SeqTable seq;
  int st = get_plan(l, B, n_q, lens_host, 1 << 30, nullptr, &plan, &kts, &seq);
  if (st != STARKV_OK) return st;
  *bytes = plan.ws_bytes;
  return STARKV_OK;
  SKV_GUARD_END
}

int starkv_decode_attention(const starkv_layer* l, const starkv_cache* c, const void* q, int B, int n_q,
                            const int32_t* lens_host, const int32_t* lens_dev, void* out, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  SKV_GUARD_BEGIN
  if (!l || !q || !out || !ws || !lens_dev_ok(lens_dev)) return STARKV_EINVAL;
  const Layer& L = l->L;
  int st = check_decode(L, c, B, n_q, lens_host);
  if (st != STARKV_OK) return st;
  st = check_bound(L, true);
  if (st != STARKV_OK) return st;
  if (((uintptr_t)ws & 255) != 0) return STARKV_EINVAL;
  if (recon_decode(L, n_q)) {
    if (lens_dev) return STARKV_EUNSUPPORTED;
    if (ws_bytes < skv::prefill_workspace_bytes(L, B, lens_host)) return STARKV_EWORKSPACE;
    return hip_status(skv::launch_prefill(L, *c, q, B, n_q, lens_host, out, ws, stream));
  }
  skv::DecodePlan plan;
  skv::KtList kts;
  skv::SeqTable seq;
  st = get_plan(l, B, n_q, lens_host, c->T_max, ws, &plan, &kts, &seq);
  if (st != STARKV_OK) return st;
  if (ws_bytes < plan.ws_bytes) return STARKV_EWORKSPACE;
  seq.lens_dev = lens_dev;
  return hip_status(skv::launch_decode(L, plan, kts, seq, q, out, c->k_rows, c->v_tiles, stream));
  SKV_GUARD_END
}

int starkv_decode_attention_hidden(const starkv_layer* l, const starkv_cache* c, const void* x, int B, int n_q,
                                   const int32_t* lens_host, const int32_t* lens_dev, void* out, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
  SKV_GUARD_BEGIN
  if (!l || !x || !out || !ws || !lens_dev_ok(lens_dev)) return STARKV_EINVAL;
  const Layer& L = l->L;
  int st = check_decode(L, c, B, n_q, lens_host);
  if (st != STARKV_OK) return st;
  st = check_bound(L, true);
  if (st != STARKV_OK) return st;
  if (L.rope_theta > 0.f) return STARKV_EUNSUPPORTED;  // rotated keys: B_g cannot be absorbed into W_q
  if (!L.d_wqk) return STARKV_ESTATE;
  if (((uintptr_t)ws & 255) != 0) return STARKV_EINVAL;
  skv::DecodePlan plan;
  skv::KtList kts;
  skv::SeqTable seq;
  st = get_plan(l, B, n_q, lens_host, c->T_max, ws, &plan, &kts, &seq);
  if (st != STARKV_OK) return st;
  if (ws_bytes < plan.ws_bytes) return STARKV_EWORKSPACE;
  seq.lens_dev = lens_dev;
  return hip_status(skv::launch_decode(L, plan, kts, seq, x, out, c->k_rows, c->v_tiles, stream, L.d_wqk));
  SKV_GUARD_END
}

int starkv_decode_step(const starkv_layer* l, const starkv_cache* c, const void* X_new, const void* q, int B,
                       int n_q, const int32_t* lens_host, const int32_t* lens_dev, void* out, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  SKV_GUARD_BEGIN
  if (!l || !q || !out || !ws || !X_new || !lens_dev_ok(lens_dev)) return STARKV_EINVAL;
  const Layer& L = l->L;
  int st = check_decode(L, c, B, n_q, lens_host);
  if (st != STARKV_OK) return st;
  st = check_bound(L, true);
  if (st != STARKV_OK) return st;
  if (((uintptr_t)ws & 255) != 0) return STARKV_EINVAL;
  int32_t lens_pre[STARKV_MAX_BATCH];
  for (int b = 0; b < B; ++b) lens_pre[b] = lens_host[b] - n_q;
  if (recon_decode(L, n_q)) {
    if (lens_dev) return STARKV_EUNSUPPORTED;
    if (ws_bytes < skv::prefill_workspace_bytes(L, B, lens_host)) return STARKV_EWORKSPACE;
    const hipError_t e = skv::launch_append(L, *c, X_new, B, n_q, lens_pre, stream);
    if (e != hipSuccess) return STARKV_EHIP;
    return hip_status(skv::launch_prefill(L, *c, q, B, n_q, lens_host, out, ws, stream));
  }
  skv::DecodePlan plan;
  skv::KtList kts;
  skv::SeqTable seq;
  st = get_plan(l, B, n_q, lens_host, c->T_max, ws, &plan, &kts, &seq);
  if (st != STARKV_OK) return st;
  if (ws_bytes < plan.ws_bytes) return STARKV_EWORKSPACE;
  seq.lens_dev = lens_dev;
  return hip_status(skv::launch_step(L, *c, plan, kts, seq, X_new, lens_pre, q, out, stream));
  SKV_GUARD_END
}

int starkv_layer_set_rope(starkv_layer* l, float theta, int rotary_dim) {
  if (!l) return STARKV_EINVAL;
  Layer& L = l->L;
  if (rotary_dim == 0) {
    L.rope_theta = 0.f;
    L.rotary_dim = 0;
    return STARKV_OK;
  }
  if (rotary_dim < 0 || rotary_dim > L.d_h || bad_float(theta) || !(theta > 0.f)) return STARKV_EINVAL;
  if (rotary_dim != L.d_h || L.d_h % 64 != 0 || L.dtype != STARKV_BF16) return STARKV_EUNSUPPORTED;
  L.rope_theta = theta;
  L.rotary_dim = rotary_dim;
  return skv::layer_write_rope(&L);  // (no-op until the layer's device tables exist)
}

static int check_prefill(const Layer& L, const starkv_cache* c, int B, int n_q, const int32_t* lens) {
  if (!lens || B <= 0 || n_q <= 0) return STARKV_EINVAL;
  if (B > STARKV_MAX_BATCH) return STARKV_EUNSUPPORTED;
  if (L.dtype != STARKV_BF16) return STARKV_EUNSUPPORTED;
  if (c) {
    const int st = check_cache(L, c, B);
    if (st != STARKV_OK) return st;
  }
  long total = 0;
  for (int b = 0; b < B; ++b) {
    if (lens[b] < n_q) return STARKV_EINVAL;
    if (c && lens[b] > c->T_max) return STARKV_ECAPACITY;
    total += (lens[b] + STARKV_TILE_TOKENS - 1) / STARKV_TILE_TOKENS * STARKV_TILE_TOKENS;
  }
  if (total > (1L << 30) / (L.n_lat > L.H_kv * L.d_h ? L.n_lat : L.H_kv * L.d_h)) return STARKV_EUNSUPPORTED;
  return STARKV_OK;
}

int starkv_prefill_workspace_bytes(const starkv_layer* l, int B, int n_q, const int32_t* lens_host, size_t* bytes) {
  SKV_GUARD_BEGIN
  if (!l || !bytes) return STARKV_EINVAL;
  const int st = check_prefill(l->L, nullptr, B, n_q, lens_host);
  if (st != STARKV_OK) return st;
  *bytes = skv::prefill_workspace_bytes(l->L, B, lens_host);
  return STARKV_OK;
  SKV_GUARD_END
}

int starkv_prefill_attention(const starkv_layer* l, const starkv_cache* c, const void* q, int B, int n_q,
                             const int32_t* lens_host, void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  SKV_GUARD_BEGIN
  if (!l || !q || !out || !ws) return STARKV_EINVAL;
  const Layer& L = l->L;
  int st = check_prefill(L, c, B, n_q, lens_host);
  if (st != STARKV_OK) return st;
  st = check_bound(L, true);
  if (st != STARKV_OK) return st;
  if (((uintptr_t)ws & 255) != 0) return STARKV_EINVAL;
  if (ws_bytes < skv::prefill_workspace_bytes(L, B, lens_host)) return STARKV_EWORKSPACE;
  return hip_status(skv::launch_prefill(L, *c, q, B, n_q, lens_host, out, ws, stream));
  SKV_GUARD_END
}

int starkv_decode_step_noalloc(const starkv_layer* l, const starkv_cache* c, const void* X_new, const void* q,
                               int B, int n_q, const int32_t* lens_host, const int32_t* lens_dev, void* out,
                               hipStream_t stream) {
  SKV_GUARD_BEGIN
  if (!l || !q || !out || !X_new || !lens_dev_ok(lens_dev)) return STARKV_EINVAL;
  const Layer& L = l->L;
  int st = check_decode(L, c, B, n_q, lens_host);
  if (st != STARKV_OK) return st;
  st = check_bound(L, true);
  if (st != STARKV_OK) return st;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != STARKV_OK) return st;
  int32_t lens_pre[STARKV_MAX_BATCH];
  for (int b = 0; b < B; ++b) lens_pre[b] = lens_host[b] - n_q;
  if (recon_decode(L, n_q)) {
    if (lens_dev) return STARKV_EUNSUPPORTED;
    if (skv::prefill_workspace_bytes(L, B, lens_host) > kScratchBytes) return STARKV_EWORKSPACE;
    const hipError_t e = skv::launch_append(L, *c, X_new, B, n_q, lens_pre, stream);
    if (e != hipSuccess) return STARKV_EHIP;
    return hip_status(skv::launch_prefill(L, *c, q, B, n_q, lens_host, out, ws, stream));
  }
  skv::DecodePlan plan;
  skv::KtList kts;
  skv::SeqTable seq;
  st = get_plan(l, B, n_q, lens_host, c->T_max, ws, &plan, &kts, &seq);
  if (st != STARKV_OK) return st;
  if (plan.ws_bytes > kScratchBytes) return STARKV_EWORKSPACE;
  seq.lens_dev = lens_dev;
  return hip_status(skv::launch_step(L, *c, plan, kts, seq, X_new, lens_pre, q, out, stream));
  SKV_GUARD_END
}

int starkv_reconstruct(const starkv_layer* l, const starkv_cache* c, int b, int t0, int t1, void* K_out,
                       void* V_out, hipStream_t stream) {
  SKV_GUARD_BEGIN
  if (!l) return STARKV_EINVAL;
  int st = check_cache(l->L, c, 1);
  if (st != STARKV_OK) return st;
  if (b < 0 || b >= c->B || t0 < 0 || t1 < t0 || t1 > c->T_max) return STARKV_EINVAL;
  if (t0 == t1) return STARKV_OK;
  if (!K_out || !V_out) return STARKV_EINVAL;
  st = check_bound(l->L, true);
  if (st != STARKV_OK) return st;
  return hip_status(skv::launch_reconstruct(l->L, *c, b, t0, t1, K_out, V_out, stream));
  SKV_GUARD_END
}

int starkv_profile_enable(int on) { return skv::profile_enable(on); }

int starkv_profile_read(starkv_kernel_time* out, int max_entries, int* n_entries, int reset) {
  SKV_GUARD_BEGIN
  if (max_entries < 0 || (max_entries > 0 && !out)) return STARKV_EINVAL;
  return skv::profile_read(out, max_entries, n_entries, reset) == 0 ? STARKV_OK : STARKV_EHIP;
  SKV_GUARD_END
}

}  // extern "C"
