// Kernels of table row 8 (see mg_table.h).
#include "mg_launch.h"

MG_DEFINE_ROW(8, Cfg8, Fast8)
