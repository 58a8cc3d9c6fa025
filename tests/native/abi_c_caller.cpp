// A plain C++ caller of the library's C ABI (include/e2d2_attn.h): device memory from
// hipMalloc, the null stream, no Python and no torch.  Built with the host compiler and
// run by tests/test_gpu_c_abi.py on a GPU.
//
// Checks, each against a closed form that the masks' definitions fix
// ([Notes] "Encoder-Decoder Diffusion Language Models for Efficient Training and
// Inference", Paper-Notes page, 方法详解 §3 采样算法 and §4 训练算法):
//   * argument validation returns its status before anything touches the GPU;
//   * with all queries zero every score is 0, so each output row is the mean of the
//     value rows its mask allows and LSE = ln(number of allowed keys): encoder
//     (keys of the own and earlier blocks), decoder (clean keys of earlier blocks plus
//     the noised keys of the own block), denoising step (all cached rows plus the own
//     block);
//   * the KV-cache append writes the new rows bitwise and leaves the others alone.
// Prints one line per failed check and a summary; exit status 0 when all pass.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "e2d2_attn.h"

namespace {

int g_checks = 0, g_fails = 0;

void expect(bool ok, const char* what, double got = 0, double want = 0) {
  ++g_checks;
  if (!ok) {
    ++g_fails;
    std::printf("FAIL %s (got %.6g, want %.6g)\n", what, got, want);
  }
}

#define HIP_OK(call)                                                         \
  do {                                                                       \
    hipError_t e_ = (call);                                                  \
    if (e_ != hipSuccess) {                                                  \
      std::printf("FAIL %s: hip error %d\n", #call, (int)e_);                \
      return 1;                                                              \
    }                                                                        \
  } while (0)

// bf16 <-> float, round to nearest even (finite values only).
uint16_t to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
float from_bf16(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Deterministic values in [-1, 1) (xorshift64*).
struct Rng {
  uint64_t s;
  float next() {
    s ^= s >> 12;
    s ^= s << 25;
    s ^= s >> 27;
    return (float)((s * 2685821657736338717ull) >> 40) / (float)(1u << 23) - 1.0f;
  }
};

// A host tensor of n values in the library's element type (bf16 or fp32), with its
// float values kept for the reference.
struct Host {
  int dtype;
  std::vector<float> val;
  std::vector<uint16_t> bf;
  Host(int dt, size_t n, Rng* rng) : dtype(dt), val(n, 0.f), bf(dt == E2D2_BF16 ? n : 0) {
    for (size_t i = 0; i < n; ++i) {
      float x = rng != nullptr ? rng->next() : 0.f;
      if (dt == E2D2_BF16) {
        bf[i] = to_bf16(x);
        x = from_bf16(bf[i]);
      }
      val[i] = x;
    }
  }
  size_t bytes() const { return val.size() * (dtype == E2D2_BF16 ? 2 : 4); }
  const void* data() const {
    return dtype == E2D2_BF16 ? (const void*)bf.data() : (const void*)val.data();
  }
};

void* upload(const Host& h) {
  void* p = nullptr;
  if (hipMalloc(&p, h.bytes()) != hipSuccess) return nullptr;
  if (hipMemcpy(p, h.data(), h.bytes(), hipMemcpyHostToDevice) != hipSuccess) return nullptr;
  return p;
}

// Device -> host copy of n elements as floats; a failed copy counts as a failed check.
std::vector<float> download(const void* p, size_t n, int dtype) {
  std::vector<float> out(n, NAN);
  hipError_t e;
  if (dtype == E2D2_BF16) {
    std::vector<uint16_t> b(n);
    e = hipMemcpy(b.data(), p, n * 2, hipMemcpyDeviceToHost);
    for (size_t i = 0; i < n; ++i) out[i] = from_bf16(b[i]);
  } else {
    e = hipMemcpy(out.data(), p, n * 4, hipMemcpyDeviceToHost);
  }
  expect(e == hipSuccess, "device to host copy", (double)e, 0);
  return out;
}

// Compares output row (b, h, i) with the mean of value rows `keys` of the two value
// sources and the LSE with ln(count).
struct RowCheck {
  int dtype, d;
  double tol() const { return dtype == E2D2_BF16 ? 2e-2 : 1e-5; }
  void row(const char* what, const float* o_row, float lse, const std::vector<const float*>& v_rows) {
    const double n = (double)v_rows.size();
    double worst = 0, got = 0, want = 0;
    for (int c = 0; c < d; ++c) {
      double m = 0;
      for (const float* v : v_rows) m += v[c];
      m /= n;
      const double err = std::fabs(o_row[c] - m);
      if (err > worst) {
        worst = err;
        got = o_row[c];
        want = m;
      }
    }
    expect(worst <= tol() * std::fmax(1.0, std::fabs(want)), what, got, want);
    expect(std::fabs(lse - std::log(n)) <= 1e-3 * std::fmax(1.0, std::log(n)), what, lse, std::log(n));
  }
};

int training_checks(int dtype) {
  const int B = 1, H = 2, L = 100, S = 7, d = 64;
  const float scale = 0.125f;
  const size_t n = (size_t)B * H * L * d;
  Rng rng{0x5EED0001ull + (uint64_t)dtype};
  Host q(dtype, n, nullptr), kc(dtype, n, &rng), vc(dtype, n, &rng), kd(dtype, n, &rng),
      vd(dtype, n, &rng);
  void *dq = upload(q), *dkc = upload(kc), *dvc = upload(vc), *dkd = upload(kd), *dvd = upload(vd);
  void *denc = nullptr, *ddec = nullptr;
  float *lenc = nullptr, *ldec = nullptr;
  HIP_OK(hipMalloc(&denc, q.bytes()));
  HIP_OK(hipMalloc(&ddec, q.bytes()));
  HIP_OK(hipMalloc((void**)&lenc, (size_t)B * H * L * 4));
  HIP_OK(hipMalloc((void**)&ldec, (size_t)B * H * L * 4));
  if (!dq || !dkc || !dvc || !dkd || !dvd) return 1;

  // validation happens before any launch
  expect(e2d2_attn_train_fwd(dtype, B, H, H, L, d, S, scale, nullptr, dkc, dvc, dkd, dvd, ddec,
                             ldec, nullptr, nullptr, nullptr, nullptr, nullptr) == E2D2_ERR_NULL,
         "train_fwd: NULL q_dec is E2D2_ERR_NULL");
  expect(e2d2_attn_train_fwd(dtype, B, H, H, L, d, 0, scale, dq, dkc, dvc, dkd, dvd, ddec, ldec,
                             nullptr, nullptr, nullptr, nullptr, nullptr) == E2D2_ERR_SHAPE,
         "train_fwd: S = 0 is E2D2_ERR_SHAPE");
  expect(e2d2_attn_encoder_blockcausal(dtype, B, H, H, L, 48, S, scale, dq, dkc, dvc, denc, lenc,
                                       nullptr, nullptr) == E2D2_ERR_UNSUPPORTED,
         "encoder: d = 48 is E2D2_ERR_UNSUPPORTED");

  // encoder and decoder, one launch each
  expect(e2d2_attn_encoder_blockcausal(dtype, B, H, H, L, d, S, scale, dq, dkc, dvc, denc, lenc,
                                       nullptr, nullptr) == E2D2_OK,
         "encoder call");
  expect(e2d2_attn_train_fwd(dtype, B, H, H, L, d, S, scale, dq, dkc, dvc, dkd, dvd, ddec, ldec,
                             nullptr, nullptr, nullptr, nullptr, nullptr) == E2D2_OK,
         "decoder call");
  HIP_OK(hipDeviceSynchronize());
  const std::vector<float> oe = download(denc, n, dtype), od = download(ddec, n, dtype);
  std::vector<float> le((size_t)B * H * L), ld((size_t)B * H * L);
  HIP_OK(hipMemcpy(le.data(), lenc, le.size() * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(ld.data(), ldec, ld.size() * 4, hipMemcpyDeviceToHost));

  RowCheck rc{dtype, d};
  for (int h = 0; h < H; ++h) {
    const size_t base = (size_t)h * L * d;
    for (int i = 0; i < L; ++i) {
      const int b0 = (i / S) * S, b1 = std::min(L, b0 + S);
      std::vector<const float*> enc_rows, dec_rows;
      for (int j = 0; j < b1; ++j) enc_rows.push_back(&vc.val[base + (size_t)j * d]);
      for (int j = 0; j < b0; ++j) dec_rows.push_back(&vc.val[base + (size_t)j * d]);
      for (int j = b0; j < b1; ++j) dec_rows.push_back(&vd.val[base + (size_t)j * d]);
      rc.row(dtype == E2D2_BF16 ? "bf16 encoder row" : "f32 encoder row", &oe[base + (size_t)i * d],
             le[(size_t)h * L + i], enc_rows);
      rc.row(dtype == E2D2_BF16 ? "bf16 decoder row" : "f32 decoder row", &od[base + (size_t)i * d],
             ld[(size_t)h * L + i], dec_rows);
    }
  }
  for (void* p : {dq, dkc, dvc, dkd, dvd, denc, ddec, (void*)lenc, (void*)ldec}) (void)hipFree(p);
  return 0;
}

int denoise_checks() {
  const int B = 2, Hq = 4, Hkv = 2, S = 8, d = 128, dt = E2D2_BF16;
  const long long C = 300, cap = 320;
  const float scale = 0.08838834764831845f;
  Rng rng{0x5EED0002ull};
  Host q(dt, (size_t)B * Hq * S * d, nullptr);
  Host kc(dt, (size_t)B * Hkv * cap * d, &rng), vc(dt, (size_t)B * Hkv * cap * d, &rng);
  Host kb(dt, (size_t)B * Hkv * S * d, &rng), vb(dt, (size_t)B * Hkv * S * d, &rng);
  void *dq = upload(q), *dkc = upload(kc), *dvc = upload(vc), *dkb = upload(kb), *dvb = upload(vb);
  if (!dq || !dkc || !dvc || !dkb || !dvb) return 1;
  void* dout = nullptr;
  float* dlse = nullptr;
  HIP_OK(hipMalloc(&dout, q.bytes()));
  HIP_OK(hipMalloc((void**)&dlse, (size_t)B * Hq * S * 4));
  const size_t nws = e2d2_attn_denoise_workspace_bytes(dt, B, Hq, Hkv, S, d, C);
  void* ws = nullptr;
  if (nws) HIP_OK(hipMalloc(&ws, nws));
  if (nws) {
    expect(e2d2_attn_denoise_step(dt, B, Hq, Hkv, S, d, scale, dq, dkc, dvc, C, cap, dkb, dvb, dout,
                                  dlse, nullptr, 0, nullptr, nullptr) == E2D2_ERR_WORKSPACE,
           "denoise: missing workspace is E2D2_ERR_WORKSPACE");
  }
  expect(e2d2_attn_denoise_step(dt, B, Hq, Hkv, S, d, scale, dq, dkc, dvc, C, cap, dkb, dvb, dout,
                                dlse, ws, nws, nullptr, nullptr) == E2D2_OK,
         "denoise call");
  HIP_OK(hipDeviceSynchronize());
  const std::vector<float> o = download(dout, q.val.size(), dt);
  std::vector<float> lse((size_t)B * Hq * S);
  HIP_OK(hipMemcpy(lse.data(), dlse, lse.size() * 4, hipMemcpyDeviceToHost));
  RowCheck rc{dt, d};
  for (int b = 0; b < B; ++b)
    for (int hq = 0; hq < Hq; ++hq) {
      const int hk = hq / (Hq / Hkv);
      std::vector<const float*> rows;
      for (long long j = 0; j < C; ++j) rows.push_back(&vc.val[(((size_t)b * Hkv + hk) * cap + j) * d]);
      for (int j = 0; j < S; ++j) rows.push_back(&vb.val[(((size_t)b * Hkv + hk) * S + j) * d]);
      for (int i = 0; i < S; ++i)
        rc.row("denoise row", &o[(((size_t)b * Hq + hq) * S + i) * d],
               lse[((size_t)b * Hq + hq) * S + i], rows);
    }

  // append: rows [C, C + S) of both caches become the new rows, bitwise
  const std::vector<float> k_before = download(dkc, kc.val.size(), dt);
  expect(e2d2_kv_cache_append(dt, B, Hkv, S, d, dkc, dvc, cap - S + 1, cap, dkb, dvb, nullptr) ==
             E2D2_ERR_CAPACITY,
         "append past the capacity is E2D2_ERR_CAPACITY");
  expect(e2d2_kv_cache_append(dt, B, Hkv, S, d, dkc, dvc, C, cap, dkb, dvb, nullptr) == E2D2_OK,
         "append call");
  HIP_OK(hipDeviceSynchronize());
  std::vector<uint16_t> k_after(kc.val.size());
  HIP_OK(hipMemcpy(k_after.data(), dkc, k_after.size() * 2, hipMemcpyDeviceToHost));
  bool same = true;
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < Hkv; ++h)
      for (long long r = 0; r < cap; ++r)
        for (int c = 0; c < d; ++c) {
          const size_t at = (((size_t)b * Hkv + h) * cap + r) * d + c;
          const uint16_t want = (r >= C && r < C + S)
                                    ? kb.bf[(((size_t)b * Hkv + h) * S + (r - C)) * d + c]
                                    : to_bf16(k_before[at]);
          same = same && k_after[at] == want;
        }
  expect(same, "append writes the new key rows bitwise and keeps the others");
  for (void* p : {dq, dkc, dvc, dkb, dvb, dout, (void*)dlse, ws}) (void)hipFree(p);
  return 0;
}

}  // namespace

int main() {
  expect(e2d2_abi_version() == E2D2_ABI_VERSION, "abi version", e2d2_abi_version(), E2D2_ABI_VERSION);
  expect(std::strlen(e2d2_status_string(E2D2_ERR_SHAPE)) > 0, "status string");
  if (training_checks(E2D2_BF16) || training_checks(E2D2_F32) || denoise_checks()) {
    std::printf("abi_c_caller: aborted after a HIP error\n");
    return 1;
  }
  std::printf("abi_c_caller: %d checks, %d failures\n", g_checks, g_fails);
  return g_fails == 0 ? 0 : 1;
}
