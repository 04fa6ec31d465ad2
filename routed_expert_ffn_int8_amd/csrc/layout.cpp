#include "layout.hpp"

#include <cstring>

namespace moe {

void pack_matrix(const MatLayout& m, const uint32_t* q, const uint16_t* s, const uint16_t* b, uint8_t* blob) {
  const int R = m.rows, C = m.cols, G = C / kGroup, W = C / 8;
  uint8_t* Q = blob + m.q_off;
  for (int rb = 0; rb < R / kRowBlock; ++rb)
    for (int g = 0; g < G; ++g)
      for (int h = 0; h < 2; ++h)
        for (int r = 0; r < kRowBlock; ++r) {
          const int row = rb * kRowBlock + r;
          const uint32_t* src = q + (size_t)row * W + g * 8 + h * 4;
          uint8_t* dst = Q + ((((size_t)rb * G + g) * 2 + h) * kRowBlock + r) * 16;
          std::memcpy(dst, src, 16);
        }
  uint32_t* SB = reinterpret_cast<uint32_t*>(blob + m.sb_off);
  for (int rb = 0; rb < R / kRowBlock; ++rb)
    for (int g = 0; g < G; ++g)
      for (int r = 0; r < kRowBlock; ++r) {
        const size_t src = (size_t)(rb * kRowBlock + r) * G + g;
        SB[((size_t)rb * G + g) * kRowBlock + r] = (uint32_t)s[src] | ((uint32_t)b[src] << 16);
      }
}

}  // namespace moe
