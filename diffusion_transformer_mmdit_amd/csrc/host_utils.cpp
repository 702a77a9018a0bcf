// Host-side helpers of the C ABI: the shifted flow-matching sigma schedule,
// position ids and the symmetric group quantiser. Plain C++ on the CPU; no
// device work.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <string>

#include "../../include/mmdit.h"

extern "C" {

// mistral.rs FLUX.1-schnell article (FluxStepper: base_shift 0.5,
// max_shift 1.15); mflux-rs card "Flow-Matching Euler" (shift mu,
// sigma_terminal) and the telemetry table (t -> 1 limit, strict monotonicity).
int mmdit_schedule(int32_t n_steps, int32_t img_len, double base_shift, double max_shift,
                   double sigma_terminal, int32_t shift, double* sigmas) {
  if (!sigmas) return MMDIT_ERR_NULL;
  if (n_steps < 1 || img_len < 1) return MMDIT_ERR_SHAPE;
  if (!(sigma_terminal >= 0.0 && sigma_terminal < 1.0)) return MMDIT_ERR_SHAPE;
  const double mu = shift ? base_shift + (max_shift - base_shift) * (double)(img_len - 256) / (double)(4096 - 256) : 0.0;
  const double em = std::exp(mu);
  for (int i = 0; i < n_steps; ++i) {
    const double t = 1.0 - (double)i / (double)n_steps;
    sigmas[i] = em / (em + (1.0 / t - 1.0));
  }
  sigmas[n_steps] = 0.0;
  if (sigma_terminal > 0.0 && n_steps >= 2) {
    const double off_last = 1.0 - sigmas[n_steps - 1];
    const double f = (1.0 - sigma_terminal) / off_last;
    for (int i = 0; i < n_steps; ++i) sigmas[i] = 1.0 - (1.0 - sigmas[i]) * f;
  }
  return MMDIT_OK;
}

// mflux-rs RoPE visualiser: axis 0 frame, axis 1 row, axis 2 column.
int mmdit_make_ids(int32_t grid_h, int32_t grid_w, int32_t txt_len, int32_t frame, int32_t* ids) {
  if (!ids) return MMDIT_ERR_NULL;
  if (grid_h < 1 || grid_w < 1 || txt_len < 0) return MMDIT_ERR_SHAPE;
  std::memset(ids, 0, sizeof(int32_t) * 3 * (size_t)txt_len);
  for (int r = 0; r < grid_h; ++r)
    for (int c = 0; c < grid_w; ++c) {
      int32_t* p = ids + 3 * ((size_t)txt_len + (size_t)r * grid_w + c);
      p[0] = frame;
      p[1] = r;
      p[2] = c;
    }
  return MMDIT_OK;
}

static uint32_t f32_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}
static float bits_f32(uint32_t u) {
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// stable-diffusion.rs README: weights held as packed bits at rest (4-bit and
// 8-bit). Per row and group of 64 k, in float32: s = smallest bf16 >=
// max|w| / qmax, q = round-half-even(w / s), so |q| <= qmax without clamping.
// float -> bf16 bits, round to nearest even (finite inputs)
static uint16_t bf16_rne(float f) {
  const uint32_t u = f32_bits(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Sub-byte formats, groups of 128 along k: absmean scale, sign or ternary codes.
static int quantise_g128(const float* w, int32_t n_out, int32_t k_in, int32_t bits, uint8_t* out,
                         uint16_t* scales_bf16) {
  if (n_out < 1 || k_in < 128 || k_in % 128) return MMDIT_ERR_SHAPE;
  const int groups = k_in / 128;
  const size_t row_bytes = bits == 1 ? (size_t)k_in / 8 : (size_t)k_in / 4;
  std::memset(out, 0, (size_t)n_out * row_bytes);
  for (int n = 0; n < n_out; ++n) {
    for (int gi = 0; gi < groups; ++gi) {
      const float* wg = w + (size_t)n * k_in + (size_t)gi * 128;
      double sum = 0.0;
      for (int j = 0; j < 128; ++j) sum += std::fabs((double)wg[j]);
      const uint16_t sb = bf16_rne((float)(sum / 128.0));
      scales_bf16[(size_t)n * groups + gi] = sb;
      const double s = (double)bits_f32((uint32_t)sb << 16);
      for (int j = 0; j < 128; ++j) {
        const size_t k = (size_t)gi * 128 + j;
        uint8_t& byte = out[(size_t)n * row_bytes + (bits == 1 ? k / 8 : k / 4)];
        if (bits == 1) {
          if (wg[j] >= 0.0f) byte = (uint8_t)(byte | (1u << (k % 8)));
        } else {
          double q = 0.0;
          if (s > 0.0) {
            q = std::nearbyint((double)wg[j] / s);
            q = q > 1.0 ? 1.0 : (q < -1.0 ? -1.0 : q);
          }
          byte = (uint8_t)(byte | ((uint32_t)((int)q + 1) << (2 * (k % 4))));
        }
      }
    }
  }
  return MMDIT_OK;
}

int mmdit_quantise(const float* w, int32_t n_out, int32_t k_in, int32_t bits, void* packed,
                   uint16_t* scales_bf16) {
  if (!w || !packed || !scales_bf16) return MMDIT_ERR_NULL;
  if (bits == 1 || bits == 2) return quantise_g128(w, n_out, k_in, bits, static_cast<uint8_t*>(packed), scales_bf16);
  if (n_out < 1 || k_in < 64 || k_in % 64) return MMDIT_ERR_SHAPE;
  if (bits != 4 && bits != 8) return MMDIT_ERR_DTYPE;
  const float qmax = bits == 4 ? 7.0f : 127.0f;
  const int groups = k_in / 64;
  uint8_t* out = static_cast<uint8_t*>(packed);
  for (int n = 0; n < n_out; ++n) {
    for (int gi = 0; gi < groups; ++gi) {
      const float* wg = w + (size_t)n * k_in + (size_t)gi * 64;
      float amax = 0.0f;
      for (int j = 0; j < 64; ++j) amax = std::fmax(amax, std::fabs(wg[j]));
      const float s32 = amax / qmax;
      uint32_t u = f32_bits(s32);
      uint32_t hi = u >> 16;
      if (u & 0xFFFFu) hi += 1;  // round up to the next bf16
      const float s = bits_f32(hi << 16);
      scales_bf16[(size_t)n * groups + gi] = (uint16_t)hi;
      for (int j = 0; j < 64; ++j) {
        int q = 0;
        if (s > 0.0f) {
          float r = std::nearbyint(wg[j] / s);
          if (r > qmax) r = qmax;
          if (r < -qmax) r = -qmax;
          q = (int)r;
        }
        const size_t k = (size_t)gi * 64 + j;
        if (bits == 8) {
          out[(size_t)n * k_in + k] = (uint8_t)(int8_t)q;
        } else {
          uint8_t& byte = out[(size_t)n * (k_in / 2) + k / 2];
          const uint8_t nib = (uint8_t)(q & 0xF);
          if ((k & 1) == 0) byte = (uint8_t)((byte & 0xF0) | nib);
          else byte = (uint8_t)((byte & 0x0F) | (nib << 4));
        }
      }
    }
  }
  return MMDIT_OK;
}

}  // extern "C"
