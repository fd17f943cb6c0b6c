// Plain data types shared by the host launchers and the kernels.
#pragma once

namespace mla {

// 3D-RoPE rotation table, passed to kernels by value: per complex pair, its axis
// (0 = t, 1 = y, 2 = x) and its angular frequency (radians per position), in fp64 so
// that angles at large absolute positions keep their accuracy.
struct RopeTable {
  int n_pairs;
  int axis[64];
  double omega[64];
};

}  // namespace mla
