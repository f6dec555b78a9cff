// Kernels of table row 3 (see mg_table.h).
#include "mg_launch.h"

MG_DEFINE_ROW(3, Cfg3, Fast3)
