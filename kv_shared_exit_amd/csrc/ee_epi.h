// Output epilogues shared by the projection passes (ee_proj.hip: rows staged
// 8 at a time; ee_wide.hip: up to 64 rows on matrix cores).
#pragma once
#include "ee_internal.h"
#include "ee_device.h"

namespace ee {

// QKV epilogue for row n of sequence seq: v is this row's value, u its RoPE
// partner's (row n -/+ hd/2).  q and k are rounded to bf16, rotated in float32
// and rounded again; k and v go to the shared cache slot of the position.
__device__ __forceinline__ void qkv_out(const ProjArgs& a, int seq, int n, float v, float u) {
  const int hd = a.hd, half = hd >> 1;
  const int head = n >> a.hd_log2;
  const int e = n & (hd - 1);
  const int pos = a.lens[seq];
  if (head < a.H + a.Hkv) {
    const int i = e < half ? e : e - half;
    const float c = a.cosT[(size_t)pos * half + i], sn = a.sinT[(size_t)pos * half + i];
    const float x = bf2f(f2bf(v)), y = bf2f(f2bf(u));
    const float r = e < half ? x * c - y * sn : x * c + y * sn;  // (x1 c - x2 s, x2 c + x1 s)
    const uint16_t o = (uint16_t)f2bf(r);
    if (head < a.H) {
      a.qrot[((size_t)seq * a.H + head) * hd + e] = o;
    } else {
      const int kh = head - a.H;
      a.Kl[(((size_t)seq * a.Hkv + kh) * a.S + pos) * hd + e] = o;
      if (a.occ_l && kh == 0 && e == 0) a.occ_l[(size_t)seq * a.S + pos] += 1;
    }
  } else {
    const int vh = head - a.H - a.Hkv;
    a.Vl[(((size_t)seq * a.Hkv + vh) * a.S + pos) * hd + e] = (uint16_t)f2bf(v);
  }
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

}  // namespace ee
