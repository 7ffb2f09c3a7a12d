// TRIA statistics files (declared in include/tria.h): host-side parsing and
// encoding of the calibrated query statistics, and the two scalings applied to
// them before a pass (per-layer budget scales, a per-band mask).  No GPU work.
//
// Layout (little-endian; the pages give the magic, the versions and the fields,
// not the byte order or the order of the fields, which are a reading):
//   u32 magic 0x54524941, u32 version (1..3), u32 n_layers, u32 n_heads,
//   u32 n_kv_heads, u32 fc;  version >= 2: u32 head_dim (= 2 fc);
//   version >= 3: u32 flags (bit 0: layer budget scales follow),
//                 then f32 layer_budget_scales[n_layers] when bit 0 is set;
//   then per (layer, query head), layer-major: f32 q_mean_real[fc],
//   f32 q_mean_imag[fc], f32 q_abs_mean[fc];  version >= 2: f32 mrl[fc].
#include "tria.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "tria_host.h"

namespace {

tria_status sfail(tria_status s, const char* fmt, ...) {
  char msg[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(msg, sizeof msg, fmt, ap);
  va_end(ap);
  tria::set_last_error(msg);
  return s;
}

constexpr uint32_t kMagic = 0x54524941u;

uint32_t rd_u32(const unsigned char* p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

float rd_f32(const unsigned char* p) {
  const uint32_t u = rd_u32(p);
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

void wr_u32(unsigned char* p, uint32_t v) {
  p[0] = (unsigned char)v;
  p[1] = (unsigned char)(v >> 8);
  p[2] = (unsigned char)(v >> 16);
  p[3] = (unsigned char)(v >> 24);
}

void wr_f32(unsigned char* p, float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  wr_u32(p, u);
}

size_t header_bytes(uint32_t version, uint32_t flags, uint32_t n_layers) {
  size_t n = 6 * 4;
  if (version >= 2) n += 4;
  if (version >= 3) n += 4 + ((flags & 1u) ? (size_t)n_layers * 4 : 0);
  return n;
}

size_t record_floats(uint32_t version, uint32_t fc) { return (size_t)fc * (version >= 2 ? 4 : 3); }

}  // namespace

extern "C" {

tria_status tria_stats_parse(const void* bytes, size_t n_bytes, tria_stats_info* info, float* q_mean_re,
                             float* q_mean_im, float* q_abs_mean, float* mrl, float* layer_budget_scales) {
  if (!bytes || !info) return sfail(TRIA_EINVAL, "bytes and info must be non-NULL");
  const unsigned char* b = static_cast<const unsigned char*>(bytes);
  if (n_bytes < 24) return sfail(TRIA_ESHAPE, "%zu bytes: shorter than the header", n_bytes);
  if (rd_u32(b) != kMagic) return sfail(TRIA_EINVAL, "magic 0x%08x is not 0x%08x", rd_u32(b), kMagic);
  tria_stats_info h{};
  h.version = rd_u32(b + 4);
  if (h.version < 1 || h.version > 3) return sfail(TRIA_EINVAL, "version %u not in 1..3", h.version);
  h.n_layers = rd_u32(b + 8);
  h.n_heads = rd_u32(b + 12);
  h.n_kv_heads = rd_u32(b + 16);
  h.fc = rd_u32(b + 20);
  if (h.n_layers == 0 || h.n_heads == 0 || h.n_kv_heads == 0 || h.fc == 0 || h.n_heads % h.n_kv_heads)
    return sfail(TRIA_ESHAPE, "header: %u layers, %u heads, %u KV heads, fc %u", h.n_layers, h.n_heads,
                 h.n_kv_heads, h.fc);
  if (h.n_layers > (1u << 16) || h.n_heads > (1u << 12) || h.fc > (1u << 12))
    return sfail(TRIA_ESHAPE, "header sizes out of range");
  size_t off = 24;
  h.head_dim = 2 * h.fc;
  if (h.version >= 2) {
    if (n_bytes < off + 4) return sfail(TRIA_ESHAPE, "truncated header");
    h.head_dim = rd_u32(b + off);
    off += 4;
    if (h.head_dim != 2 * h.fc) return sfail(TRIA_ESHAPE, "head_dim %u != 2 fc (%u)", h.head_dim, 2 * h.fc);
  }
  uint32_t flags = 0;
  if (h.version >= 3) {
    if (n_bytes < off + 4) return sfail(TRIA_ESHAPE, "truncated header");
    flags = rd_u32(b + off);
    off += 4;
    if (flags & ~1u) return sfail(TRIA_EINVAL, "unknown flags 0x%x", flags);
  }
  h.has_budget_scales = (flags & 1u) ? 1 : 0;
  const size_t need = header_bytes(h.version, flags, h.n_layers) +
                      (size_t)h.n_layers * h.n_heads * record_floats(h.version, h.fc) * 4;
  if (n_bytes != need) return sfail(TRIA_ESHAPE, "%zu bytes, the header implies %zu", n_bytes, need);
  h.mrl_present = h.version >= 2 ? 1 : 0;
  *info = h;
  // layer budget scales: 1.0 unless the file carries them
  if (layer_budget_scales)
    for (uint32_t l = 0; l < h.n_layers; ++l)
      layer_budget_scales[l] = h.has_budget_scales ? rd_f32(b + off + 4 * (size_t)l) : 1.0f;
  if (h.has_budget_scales) off += 4 * (size_t)h.n_layers;
  const size_t F = h.fc;
  for (size_t r = 0; r < (size_t)h.n_layers * h.n_heads; ++r) {
    const unsigned char* rec = b + off + r * record_floats(h.version, h.fc) * 4;
    for (size_t f = 0; f < F; ++f) {
      if (q_mean_re) q_mean_re[r * F + f] = rd_f32(rec + 4 * f);
      if (q_mean_im) q_mean_im[r * F + f] = rd_f32(rec + 4 * (F + f));
      if (q_abs_mean) q_abs_mean[r * F + f] = rd_f32(rec + 4 * (2 * F + f));
      if (mrl) mrl[r * F + f] = h.version >= 2 ? rd_f32(rec + 4 * (3 * F + f)) : 0.0f;
    }
  }
  return TRIA_OK;
}

size_t tria_stats_encode(const tria_stats_info* info, const float* q_mean_re, const float* q_mean_im,
                         const float* q_abs_mean, const float* mrl, const float* layer_budget_scales, void* out,
                         size_t cap) {
  if (!info || info->version < 1 || info->version > 3 || info->n_layers == 0 || info->n_heads == 0 ||
      info->n_kv_heads == 0 || info->fc == 0 || info->n_heads % info->n_kv_heads || !q_mean_re || !q_mean_im ||
      !q_abs_mean)
    return 0;
  // the sizes the parser accepts
  if (info->n_layers > (1u << 16) || info->n_heads > (1u << 12) || info->fc > (1u << 12)) return 0;
  const uint32_t flags = (info->version >= 3 && info->has_budget_scales && layer_budget_scales) ? 1u : 0u;
  const size_t need = header_bytes(info->version, flags, info->n_layers) +
                      (size_t)info->n_layers * info->n_heads * record_floats(info->version, info->fc) * 4;
  if (!out || cap < need) return need;
  unsigned char* b = static_cast<unsigned char*>(out);
  wr_u32(b, kMagic);
  wr_u32(b + 4, info->version);
  wr_u32(b + 8, info->n_layers);
  wr_u32(b + 12, info->n_heads);
  wr_u32(b + 16, info->n_kv_heads);
  wr_u32(b + 20, info->fc);
  size_t off = 24;
  if (info->version >= 2) {
    wr_u32(b + off, 2 * info->fc);
    off += 4;
  }
  if (info->version >= 3) {
    wr_u32(b + off, flags);
    off += 4;
    if (flags)
      for (uint32_t l = 0; l < info->n_layers; ++l, off += 4) wr_f32(b + off, layer_budget_scales[l]);
  }
  const size_t F = info->fc;
  for (size_t r = 0; r < (size_t)info->n_layers * info->n_heads; ++r) {
    for (size_t f = 0; f < F; ++f, off += 4) wr_f32(b + off, q_mean_re[r * F + f]);
    for (size_t f = 0; f < F; ++f, off += 4) wr_f32(b + off, q_mean_im[r * F + f]);
    for (size_t f = 0; f < F; ++f, off += 4) wr_f32(b + off, q_abs_mean[r * F + f]);
    if (info->version >= 2)
      for (size_t f = 0; f < F; ++f, off += 4) wr_f32(b + off, mrl ? mrl[r * F + f] : 0.0f);
  }
  return need;
}

tria_status tria_stats_band_mask(int32_t n_rows, int32_t fc, const float* mask, float* q_mean_re, float* q_mean_im,
                                 float* q_abs_mean) {
  if (n_rows < 0 || fc < 1 || !mask || !q_mean_re || !q_mean_im || !q_abs_mean)
    return sfail(TRIA_EINVAL, "invalid band-mask arguments");
  for (int32_t f = 0; f < fc; ++f)
    if (!(mask[f] >= 0.0f) || !std::isfinite(mask[f])) return sfail(TRIA_EINVAL, "mask[%d] is not finite and >= 0", f);
  for (int64_t r = 0; r < n_rows; ++r)
    for (int32_t f = 0; f < fc; ++f) {
      const size_t i = (size_t)r * fc + f;
      const double re = q_mean_re[i], im = q_mean_im[i], m = mask[f];
      const double c = std::sqrt(re * re + im * im);
      q_mean_re[i] = (float)(re * m);
      q_mean_im[i] = (float)(im * m);
      // keep the norm weight E|q_f| - |E q_f| unchanged
      q_abs_mean[i] = (float)((double)q_abs_mean[i] + (m - 1.0) * c);
    }
  return TRIA_OK;
}

tria_status tria_stats_layer_budgets(int32_t n_units, const int32_t* unit_layer, int32_t n_layers,
                                     const float* layer_budget_scales, int32_t budget, int32_t* budgets) {
  if (n_units < 0 || n_layers < 1 || budget < 0 || !unit_layer || !layer_budget_scales || !budgets)
    return sfail(TRIA_EINVAL, "invalid layer-budget arguments");
  for (int32_t u = 0; u < n_units; ++u) {
    const int32_t l = unit_layer[u];
    if (l < 0 || l >= n_layers) return sfail(TRIA_EINVAL, "unit_layer[%d] = %d outside [0, %d)", u, l, n_layers);
    const float s = layer_budget_scales[l];
    if (!(s >= 0.0f) || !std::isfinite(s)) return sfail(TRIA_EINVAL, "layer_budget_scales[%d] invalid", l);
    const double v = std::floor((double)budget * s + 0.5);
    budgets[u] = v > 2147483647.0 ? 2147483647 : (int32_t)v;
  }
  return TRIA_OK;
}

}  // extern "C"
