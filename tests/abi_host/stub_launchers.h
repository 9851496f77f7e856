// What the stand-in launchers saw (see stub_launchers.cpp).
#pragma once

namespace stub {
extern int launches;
extern const void *last_ws;
extern int last_m, last_n, last_k;
}  // namespace stub
