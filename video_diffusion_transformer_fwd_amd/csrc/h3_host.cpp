// Host integer logic of the sampler: frame alignment, token grid, sigma schedule, layer
// thinning and the token-pairing plan.  Exact arithmetic only; see include/h3dit.h for the
// page citations of each rule.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <numeric>
#include <string>
#include <vector>

#include "h3_internal.h"

namespace h3 {

static thread_local std::string g_last_error;

void set_error(const std::string &msg) { g_last_error = msg; }
void clear_error() { g_last_error.clear(); }
int32_t fail(int32_t code, const std::string &msg) {
  g_last_error = msg;
  return code;
}
int32_t check_launch(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(H3_EHIP, std::string(what) + ": " + hipGetErrorString(e));
  return H3_OK;
}

}  // namespace h3

using namespace h3;

extern "C" {

const char *h3_last_error(void) { return g_last_error.c_str(); }

int32_t h3_abi_version(void) { return 104; }

int32_t h3_align_frames(int32_t requested, int32_t *frames) {
  if (!frames) return fail(H3_EINVAL, "h3_align_frames: frames is NULL");
  if (requested < 1) return fail(H3_EINVAL, "h3_align_frames: requested must be >= 1");
  // smallest 5 + 17 n >= requested, n >= 0
  int64_t n = requested <= 5 ? 0 : (static_cast<int64_t>(requested) - 5 + 16) / 17;
  int64_t f = 5 + 17 * n;
  if (f > INT32_MAX) return fail(H3_EINVAL, "h3_align_frames: request too large");
  *frames = static_cast<int32_t>(f);
  return H3_OK;
}

int32_t h3_frames_for_seconds(double seconds, int32_t *frames) {
  if (!frames) return fail(H3_EINVAL, "h3_frames_for_seconds: frames is NULL");
  if (!(seconds > 0.0)) return fail(H3_EINVAL, "h3_frames_for_seconds: seconds must be > 0");
  double req = std::ceil(24.0 * seconds);
  if (req > 2147483000.0) return fail(H3_EINVAL, "h3_frames_for_seconds: too long");
  return h3_align_frames(static_cast<int32_t>(req), frames);
}

int32_t h3_latent_frames(int32_t frames, int32_t *f_lat) {
  if (!f_lat) return fail(H3_EINVAL, "h3_latent_frames: f_lat is NULL");
  if (frames < 1) return fail(H3_EINVAL, "h3_latent_frames: frames must be >= 1");
  *f_lat = 1 + (frames - 1) / 4;
  return H3_OK;
}

int32_t h3_token_grid(int32_t width, int32_t height, int32_t reference_rope, int32_t *grid_h,
                      int32_t *grid_w, float *rope_spatial_scale) {
  if (!grid_h || !grid_w || !rope_spatial_scale)
    return fail(H3_EINVAL, "h3_token_grid: NULL output");
  if (width < 32 || height < 32 || width % 32 || height % 32)
    return fail(H3_EINVAL, "h3_token_grid: width/height must be multiples of 32 and >= 32");
  if (static_cast<int64_t>(width) * height > 768LL * 1344LL)
    return fail(H3_EINVAL, "h3_token_grid: width*height exceeds 768*1344");
  *grid_h = height / 32;
  *grid_w = width / 32;
  *rope_spatial_scale = (*grid_h == 8 && *grid_w == 8 && !reference_rope) ? 0.5f : 1.0f;
  return H3_OK;
}

int32_t h3_schedule(int32_t steps, int32_t reuse, int32_t core_reuse, float *sigmas,
                    uint8_t *fresh, int32_t *n_fresh) {
  if (!sigmas || !fresh || !n_fresh) return fail(H3_EINVAL, "h3_schedule: NULL output");
  if (steps < 1 || reuse < 1 || core_reuse < 1)
    return fail(H3_EINVAL, "h3_schedule: steps, reuse, core_reuse must be >= 1");
  if (reuse > 1 && core_reuse > 1)
    return fail(H3_EINVAL, "h3_schedule: --reuse and --core-reuse are mutually exclusive");
  if (core_reuse > 6) return fail(H3_EINVAL, "h3_schedule: core_reuse must be at most 6");
  if (steps > (1 << 20)) return fail(H3_EINVAL, "h3_schedule: steps must be at most 2^20");
  const float n = static_cast<float>(steps);
  for (int32_t i = 0; i <= steps; ++i) sigmas[i] = static_cast<float>(steps - i) / n;
  // whole-velocity reuse (reuse > 1) or core-residual reuse (core_reuse > 1): the same rule
  // marks the steps whose core runs fresh
  const int32_t r = reuse > 1 ? reuse : core_reuse;
  int32_t cnt = 0;
  for (int32_t i = 0; i < steps; ++i) {
    fresh[i] = (i % r == 0 || i == steps - 1) ? 1 : 0;
    cnt += fresh[i];
  }
  *n_fresh = cnt;
  return H3_OK;
}

static double bf16_bits_to_double(uint16_t h) {
  uint32_t u = static_cast<uint32_t>(h) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return static_cast<double>(f);
}

int32_t h3_select_layers(const uint16_t *mod_table, int32_t n_blocks, int32_t d_model,
                         int32_t n_active, int32_t *active) {
  if (!mod_table || !active) return fail(H3_EINVAL, "h3_select_layers: NULL pointer");
  if (n_blocks < 2 || d_model < 1) return fail(H3_EINVAL, "h3_select_layers: bad sizes");
  if (n_active < 2 || n_active > n_blocks)
    return fail(H3_EINVAL, "h3_select_layers: n_active must be in [2, n_blocks]");
  std::vector<double> key(n_blocks);
  for (int32_t b = 0; b < n_blocks; ++b) {
    const uint16_t *g1 = mod_table + (static_cast<size_t>(b) * 6 + 2) * d_model;
    const uint16_t *g2 = mod_table + (static_cast<size_t>(b) * 6 + 5) * d_model;
    double s = 0.0;
    for (int32_t c = 0; c < d_model; ++c) {
      s += std::fabs(bf16_bits_to_double(g1[c]));
      s += std::fabs(bf16_bits_to_double(g2[c]));
    }
    key[b] = s;
  }
  std::vector<int32_t> mid;
  for (int32_t b = 1; b < n_blocks - 1; ++b) mid.push_back(b);
  std::stable_sort(mid.begin(), mid.end(), [&](int32_t a, int32_t b) {
    if (key[a] != key[b]) return key[a] < key[b];
    return a > b;  // equal keys: the higher index is dropped first
  });
  std::vector<uint8_t> drop(n_blocks, 0);
  for (int32_t i = 0; i < n_blocks - n_active; ++i) drop[mid[i]] = 1;
  int32_t j = 0;
  for (int32_t b = 0; b < n_blocks; ++b)
    if (!drop[b]) active[j++] = b;
  return H3_OK;
}

int32_t h3_token_plan(int32_t f_lat, int32_t grid_h, int32_t grid_w, int32_t eval_index,
                      int32_t n_active, int32_t *merge_after, int32_t *restore_before,
                      int32_t *pairs, int32_t *n_reduced) {
  if (!merge_after || !restore_before || !n_reduced)
    return fail(H3_EINVAL, "h3_token_plan: NULL output");
  if (f_lat < 1 || grid_h < 1 || grid_w < 1 || eval_index < 0)
    return fail(H3_EINVAL, "h3_token_plan: bad geometry");
  if (static_cast<int64_t>(f_lat) * grid_h * grid_w > (1 << 24))
    return fail(H3_ESHAPE, "h3_token_plan: too many tokens");  // the cap of h3_geom_tokens
  if (n_active <= 3) return fail(H3_EINVAL, "h3_token_plan: needs more than 3 active blocks");
  *merge_after = 3;
  int32_t r = eval_index < 10 ? 40 : 30;
  *restore_before = std::min(r, n_active + 1);
  const int32_t wr = (grid_w + 1) / 2;
  *n_reduced = f_lat * grid_h * wr;
  if (pairs) {
    int32_t j = 0;
    for (int32_t row = 0; row < f_lat * grid_h; ++row)
      for (int32_t c = 0; c < wr; ++c) {
        int32_t a = row * grid_w + 2 * c;
        int32_t b = (2 * c + 1 < grid_w) ? a + 1 : a;
        pairs[2 * j] = a;
        pairs[2 * j + 1] = b;
        ++j;
      }
  }
  return H3_OK;
}

int32_t h3_geom_tokens(const h3_geom *geom, int32_t *n_tokens) {
  if (!geom || !n_tokens) return fail(H3_EINVAL, "h3_geom_tokens: NULL pointer");
  if (geom->f_lat < 1 || geom->grid_h < 1 || geom->grid_w < 1)
    return fail(H3_EINVAL, "h3_geom_tokens: sizes must be >= 1");
  if (!(geom->rope_spatial_scale == 1.0f || geom->rope_spatial_scale == 0.5f))
    return fail(H3_EINVAL, "h3_geom_tokens: rope_spatial_scale must be 1 or 0.5");
  if (geom->paired != 0 && geom->paired != 1)
    return fail(H3_EINVAL, "h3_geom_tokens: paired must be 0 or 1");
  const int64_t w = geom->paired ? (static_cast<int64_t>(geom->grid_w) + 1) / 2 : geom->grid_w;
  int64_t n = static_cast<int64_t>(geom->f_lat) * geom->grid_h * w;
  if (n > (1 << 24)) return fail(H3_ESHAPE, "h3_geom_tokens: too many tokens");
  *n_tokens = static_cast<int32_t>(n);
  return H3_OK;
}

}  // extern "C"
